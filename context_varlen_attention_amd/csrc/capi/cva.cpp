// C ABI of libcva (declared in include/cva.h).
//
// Plan creation is pure host work (validation, metadata, schedules).  Device
// work is: one async copy of the plan tables (cva_plan_upload), one forward
// kernel (cva_fwd) and the backward kernels (cva_bwd), all on the caller's
// stream, all arguments checked on the host first so that a failing call
// enqueues nothing (MindSpeed RFC section 3.4: validate before any operator
// call).
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <sstream>
#include <vector>

#include <hip/hip_runtime_api.h>

#include "../host/plan.hpp"
#include "../kernels/launch.hpp"

using cva::Plan;

namespace {

cva_status fail(cva_status s, const std::string& msg) {
  cva::set_error(msg);
  return s;
}

cva_status hip_fail(hipError_t e, const char* what) {
  std::ostringstream os;
  os << what << ": " << hipGetErrorString(e);
  return fail(CVA_E_HIP, os.str());
}

cva::PlanTables tables(const Plan& p) {
  const int32_t* b = (const int32_t*)p.dev;
  const cva::BlobLayout& L = p.layout;
  cva::PlanTables t;
  t.segs = b + L.segs;
  t.kv_index = b + L.kv_index;
  t.row_iv = b + L.row_iv;
  t.fwd_tiles = b + L.fwd_tiles;
  t.fwd_spans = b + L.fwd_spans;
  t.dq_tiles = b + L.dq_tiles;
  t.dq_spans = b + L.dq_spans;
  t.kv_tiles = b + L.kv_tiles;
  t.kv_spans = b + L.kv_spans;
  t.zero_rows = b + L.zero_rows;
  t.fwds_slot = b + L.fwds_slot;
  t.fwds_combine = b + L.fwds_combine;
  t.deal_start = b + L.fwd_deal_start;
  t.deal_items = b + L.fwd_deal_items;
  return t;
}

cva_status check_scale(float s) {
  if (!std::isfinite(s) || !(s > 0.f)) return fail(CVA_E_SCALE, "softmax_scale must be finite and > 0");
  return CVA_OK;
}

// Attention dropout of a call: threshold t = round(256 p) clamped to 255 (the
// random byte of a pair must be >= t to keep it) and the scale 256 / (256 - t)
// of the kept probabilities; t = 0 (p < 1/512) drops nothing.
cva_status make_drop(float p, uint64_t seed, cva::DropParams* d) {
  if (!(p >= 0.f && p < 1.f)) return fail(CVA_E_ARG, "dropout probability must be in [0, 1)");
  const int t = std::min(255, (int)std::floor(256.0 * (double)p + 0.5));
  d->t = (uint32_t)t;
  d->seed_lo = (uint32_t)(seed & 0xFFFFFFFFull);
  d->seed_hi = (uint32_t)(seed >> 32);
  d->scale = (float)(256.0 / (256.0 - t));
  return CVA_OK;
}

constexpr cva::DropParams kNoDrop{0u, 0u, 0u, 1.f};

// Event-pair timing around kernel launches (cva_timing_enable / cva_timing_read).
// One process-wide timer; its state is guarded by a mutex so that launches from
// several host threads record their events without corrupting it (each
// before/after pair is taken under one lock held across the launch).
struct Timer final : cva::LaunchHook {
  std::mutex mu;
  struct Rec { int kernel; hipEvent_t a, b; };
  std::atomic<bool> on{false};
  std::vector<Rec> pending;
  std::vector<hipEvent_t> pool;
  int64_t launches[CVA_N_KERNELS] = {};
  double total_ms[CVA_N_KERNELS] = {};
  hipEvent_t get() {
    if (!pool.empty()) { hipEvent_t e = pool.back(); pool.pop_back(); return e; }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
  uint32_t mask = ~0u;  // kernels to time
  bool skip = false;    // the launch in flight is not timed
  void before(int kernel, hipStream_t s) override {
    mu.lock();  // released in after(): the launch between them is recorded as one pair
    skip = ((mask >> kernel) & 1u) == 0;
    if (skip) return;
    Rec r{kernel, get(), get()};
    if (r.a) (void)hipEventRecord(r.a, s);
    pending.push_back(r);
  }
  void after(int, hipStream_t s) override {
    if (!skip && !pending.empty() && pending.back().b) (void)hipEventRecord(pending.back().b, s);
    mu.unlock();
  }
  hipError_t drain() {
    hipError_t err = hipSuccess;
    for (Rec& r : pending) {
      float ms = 0.f;
      if (r.a && r.b) {
        hipError_t e = hipEventSynchronize(r.b);
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.a, r.b);
        if (e != hipSuccess && err == hipSuccess) err = e;
      }
      launches[r.kernel] += 1;
      total_ms[r.kernel] += ms;
      if (r.a) pool.push_back(r.a);
      if (r.b) pool.push_back(r.b);
    }
    pending.clear();
    return err;
  }
  void reset() {
    for (int k = 0; k < CVA_N_KERNELS; ++k) { launches[k] = 0; total_ms[k] = 0.0; }
  }
};

Timer g_timer;

cva::LaunchHook* hook() { return g_timer.on ? &g_timer : nullptr; }

cva_status check_ready(const Plan* p) {
  if (p == nullptr) return fail(CVA_E_ARG, "plan is NULL");
  if (p->dev == nullptr) return fail(CVA_E_NOT_UPLOADED, "plan has no device copy; call cva_plan_upload first");
  return CVA_OK;
}

}  // namespace

extern "C" {

const char* cva_last_error(void) { return cva::last_error(); }

cva_status cva_plan_create(const int32_t* cu_seqlens, int32_t n_seqs, int32_t cp_size,
                           int32_t rank, const cva_mask_desc* mask, int32_t hq, int32_t hkv,
                           int32_t d_qk, int32_t d_v, int32_t dtype, cva_plan** out) {
  cva::set_error("");
  if (out == nullptr) return fail(CVA_E_ARG, "out is NULL");
  *out = nullptr;
  cva_status st = cva::validate_request(cu_seqlens, n_seqs, cp_size, rank, mask, hq, hkv, d_qk,
                                        d_v, dtype);
  if (st != CVA_OK) return st;
  Plan* p = new (std::nothrow) Plan();
  if (p == nullptr) return fail(CVA_E_ARG, "out of host memory");
  try {
    p->n_seqs = n_seqs;
    p->cp_size = cp_size;
    p->rank = rank;
    p->hq = hq;
    p->hkv = hkv;
    p->d_qk = d_qk;
    p->d_v = d_v;
    p->dtype = dtype;
    p->cu.assign(cu_seqlens, cu_seqlens + n_seqs + 1);
    if (mask != nullptr) {
      p->mask_type = mask->type;
      p->sink = mask->sink;
      p->window = mask->window;
      if (mask->type == CVA_MASK_BLOCKWISE) p->block = mask->block;
      if (mask->type == CVA_MASK_SHARED_PREFIX) {
        p->n_branches = mask->n_branches;
        const size_t nb = (size_t)n_seqs * (mask->n_branches + 1);
        p->branch_bounds.assign(mask->branch_bounds, mask->branch_bounds + nb);
      }
    }
    st = cva::build_metadata(*p);
    if (st == CVA_OK) st = cva::build_schedules(*p);
    if (st == CVA_OK) cva::build_blob(*p);
  } catch (const std::bad_alloc&) {
    st = fail(CVA_E_ARG, "out of host memory while building the plan");
  }
  if (st != CVA_OK) {
    delete p;
    return st;
  }
  *out = reinterpret_cast<cva_plan*>(p);
  return CVA_OK;
}

void cva_plan_destroy(cva_plan* plan) {
  Plan* p = reinterpret_cast<Plan*>(plan);
  if (p != nullptr && p->upload_done != nullptr) {
    // an upload may still be reading the host tables: let it finish first
    (void)hipEventSynchronize((hipEvent_t)p->upload_done);
    (void)hipEventDestroy((hipEvent_t)p->upload_done);
  }
  delete p;
}

cva_status cva_plan_get_metadata(const cva_plan* plan, cva_metadata* out) {
  const Plan* p = reinterpret_cast<const Plan*>(plan);
  if (p == nullptr || out == nullptr) return fail(CVA_E_ARG, "plan or out is NULL");
  if (p->placed) return fail(CVA_E_UNSUPPORTED, "a placement share has no context-parallel metadata");
  out->local_tokens = p->T_loc;
  out->global_tokens = p->T;
  out->n_seqs = p->n_seqs;
  out->n_segments = 2 * p->n_seqs;
  out->cp_size = p->cp_size;
  out->rank = p->rank;
  out->local_cu = p->local_cu.data();
  out->actual_seq_qlen = p->aq.data();
  out->actual_seq_kvlen = p->akv.data();
  out->kv_index = p->kv_index.data();
  out->seg_q_pos0 = p->seg_q_pos0.data();
  out->kv_index_len = (int64_t)p->kv_index.size();
  out->workload_per_rank = p->workload.data();
  out->visible_pairs = p->visible_pairs;
  out->fwd_tiles = p->fwd.tile_pairs;
  out->visible_pairs_per_rank = p->visible_pairs_per_rank.data();
  return CVA_OK;
}

size_t cva_plan_device_bytes(const cva_plan* plan) {
  const Plan* p = reinterpret_cast<const Plan*>(plan);
  return p == nullptr ? 0 : (size_t)p->layout.total * sizeof(int32_t);
}

cva_status cva_plan_upload(cva_plan* plan, void* dev_buf, size_t bytes, void* stream) {
  Plan* p = reinterpret_cast<Plan*>(plan);
  if (p == nullptr || dev_buf == nullptr) return fail(CVA_E_ARG, "plan or dev_buf is NULL");
  const size_t need = (size_t)p->layout.total * sizeof(int32_t);
  if (bytes < need) {
    std::ostringstream os;
    os << "device buffer too small: " << bytes << " < " << need;
    return fail(CVA_E_ARG, os.str());
  }
  if (((uintptr_t)dev_buf) % 256 != 0) return fail(CVA_E_ARG, "device buffer must be 256-byte aligned");
  if (p->upload_done == nullptr) {
    hipEvent_t ev = nullptr;
    hipError_t e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
    if (e != hipSuccess) return hip_fail(e, "hipEventCreateWithFlags(plan upload)");
    p->upload_done = ev;
  }
  // the copy reads the plan's own host tables, which stay alive until it has
  // completed (cva_plan_destroy waits for the event): no host synchronisation
  hipError_t e = hipMemcpyAsync(dev_buf, p->blob.data(), need, hipMemcpyHostToDevice,
                                (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(plan)");
  e = hipEventRecord((hipEvent_t)p->upload_done, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord(plan upload)");
  p->dev = dev_buf;
  p->dev_bytes = bytes;
  return CVA_OK;
}

namespace {

bool splits(const Plan& p) { return p.n_split_slots > 0 && p.dtype != CVA_FP32; }

size_t split_bytes(const Plan& p) {
  if (!splits(p)) return 0;
  const size_t rows = (size_t)p.n_split_slots * p.hq * p.fwds.tile_q;  // (slot, head, row)
  const size_t o_bytes = (rows * p.d_v * sizeof(float) + 255) / 256 * 256;
  return o_bytes + rows * sizeof(float);
}

// Work-groups per head group of the streamed forward for the schedule being
// launched (its deal), or 0 for one work-group per item.  Measured on MI355X,
// the streamed form wins at Q/K head dim 192 (the 32k expanded-MLA batch:
// forward 571 -> 506 us) and loses at 128 (4-26 % on the other batches), so it
// is the default for head dims above 128 only; CVA_FWD_STREAM=1 / =0 in the
// environment selects it / one work-group per item for every plan.
int32_t stream_wgs(const Plan& p, const cva::StreamDeal& d) {
  if (const char* v = std::getenv("CVA_FWD_STREAM")) {
    if (v[0] == '0' && v[1] == 0) return 0;
    if (v[0] == '1' && v[1] == 0) return d.wgs;
  }
  return p.d_qk > 128 ? d.wgs : 0;
}

cva_status run_fwd(const Plan* p, const void* q, const void* k_rm, const void* v_rm, void* o,
                   float* lse, float softmax_scale, void* workspace, size_t ws_bytes,
                   bool split, const cva::DropParams& drop, void* stream) {
  cva_status st = check_ready(p);
  if (st != CVA_OK) return st;
  if (q == nullptr || k_rm == nullptr || v_rm == nullptr || o == nullptr || lse == nullptr)
    return fail(CVA_E_ARG, "a tensor pointer is NULL");
  if ((st = check_scale(softmax_scale)) != CVA_OK) return st;
  if (p->placed && !split)
    return fail(CVA_E_UNSUPPORTED, "a placement share runs through cva_fwd_split (its blocks merge by LSE)");
  split = split && splits(*p);
  if (split) {
    const size_t need = split_bytes(*p);
    if (workspace == nullptr || ws_bytes < need) {
      std::ostringstream os;
      os << "forward workspace needs " << need << " bytes";
      return fail(CVA_E_WORKSPACE, os.str());
    }
    if (((uintptr_t)workspace & 255) != 0) return fail(CVA_E_WORKSPACE, "forward workspace must be 256-byte aligned");
  }
  cva::FwdParams fp;
  fp.q = q;
  fp.k = k_rm;
  fp.v = v_rm;
  fp.o = o;
  fp.lse = lse;
  fp.t = tables(*p);
  fp.n_tiles = p->fwd.n_tiles();
  fp.heads_per_tile = p->fwd_heads_per_tile;
  fp.n_head_groups = p->hq / p->fwd_heads_per_tile;
  fp.hq = p->hq;
  fp.hkv = p->hkv;
  fp.group = p->hq / p->hkv;
  fp.t_loc = (int32_t)p->T_loc;
  fp.tile_q = p->fwd.tile_q;
  fp.tile_kv = p->fwd.tile_kv;
  fp.scale_log2 = softmax_scale * 1.4426950408889634f;
  fp.slot = nullptr;
  fp.ws_o = nullptr;
  fp.ws_lse = nullptr;
  fp.combine = nullptr;
  fp.n_combine = 0;
  if (split) {
    const int32_t* b = (const int32_t*)p->dev;
    fp.t.fwd_tiles = b + p->layout.fwds_tiles;
    fp.t.fwd_spans = b + p->layout.fwds_spans;
    fp.t.deal_start = b + p->layout.fwds_deal_start;
    fp.t.deal_items = b + p->layout.fwds_deal_items;
    fp.n_tiles = p->fwds.n_tiles();
    fp.slot = fp.t.fwds_slot;
    fp.combine = fp.t.fwds_combine;
    fp.n_combine = (int32_t)(p->fwds_combine.size() / cva::CB_INTS);
    const size_t rows = (size_t)p->n_split_slots * p->hq * p->fwds.tile_q;
    fp.ws_o = (float*)workspace;
    fp.ws_lse = (float*)((char*)workspace + (rows * p->d_v * sizeof(float) + 255) / 256 * 256);
  }
  fp.stream_wgs = stream_wgs(*p, split ? p->fwds_deal : p->fwd_deal);
  fp.drop = drop;
  if (drop.t != 0) fp.stream_wgs = 0;  // dropout runs one work-group per item
  hipError_t e = cva::launch_fwd(p->dtype, p->d_qk, p->d_v, fp, (hipStream_t)stream, hook());
  if (e != hipSuccess) return hip_fail(e, "forward launch");
  return CVA_OK;
}

}  // namespace

cva_status cva_fwd(const cva_plan* plan, const void* q, const void* k_rm, const void* v_rm,
                   void* o, float* lse, float softmax_scale, void* stream) {
  return run_fwd(reinterpret_cast<const Plan*>(plan), q, k_rm, v_rm, o, lse, softmax_scale,
                 nullptr, 0, false, kNoDrop, stream);
}

size_t cva_fwd_workspace_bytes(const cva_plan* plan) {
  const Plan* p = reinterpret_cast<const Plan*>(plan);
  return p == nullptr ? 0 : split_bytes(*p);
}

cva_status cva_fwd_split(const cva_plan* plan, const void* q, const void* k_rm, const void* v_rm,
                         void* o, float* lse, float softmax_scale, void* workspace,
                         size_t ws_bytes, void* stream) {
  return run_fwd(reinterpret_cast<const Plan*>(plan), q, k_rm, v_rm, o, lse, softmax_scale,
                 workspace, ws_bytes, true, kNoDrop, stream);
}

cva_status cva_fwd_dropout(const cva_plan* plan, const void* q, const void* k_rm, const void* v_rm,
                           void* o, float* lse, float softmax_scale, float dropout_p, uint64_t seed,
                           void* workspace, size_t ws_bytes, void* stream) {
  cva::DropParams d;
  cva_status st = make_drop(dropout_p, seed, &d);
  if (st != CVA_OK) return st;
  return run_fwd(reinterpret_cast<const Plan*>(plan), q, k_rm, v_rm, o, lse, softmax_scale,
                 workspace, ws_bytes, workspace != nullptr, d, stream);
}

size_t cva_bwd_workspace_bytes(const cva_plan* plan) {
  const Plan* p = reinterpret_cast<const Plan*>(plan);
  if (p == nullptr) return 0;
  return 2 * (size_t)p->T_loc * p->hq * sizeof(float);  // Delta, LSE * log2(e)
}

namespace {

cva_status check_bwd_args(const Plan* p, const void* q, const void* k_rm, const void* v_rm,
                          const void* o, const float* lse, const void* dout, void* dq,
                          void* dk_rm, void* dv_rm, float softmax_scale) {
  cva_status st = check_ready(p);
  if (st != CVA_OK) return st;
  if (q == nullptr || k_rm == nullptr || v_rm == nullptr || o == nullptr || lse == nullptr ||
      dout == nullptr || dq == nullptr || dk_rm == nullptr || dv_rm == nullptr)
    return fail(CVA_E_ARG, "a tensor pointer is NULL");
  if ((st = check_scale(softmax_scale)) != CVA_OK) return st;
  if (p->dtype == CVA_FP32) return fail(CVA_E_UNSUPPORTED, "backward is implemented for bf16 and fp16");
  if (p->placed) return fail(CVA_E_UNSUPPORTED, "the backward of a placement share is not implemented");
  return CVA_OK;
}

// Launches the backward with Delta / LSE*log2(e) in `stats` (2 * T_loc * Hq floats).
cva_status run_bwd(const Plan* p, const void* q, const void* k_rm, const void* v_rm,
                   const void* o, const float* lse, const void* dout, void* dq, void* dk_rm,
                   void* dv_rm, float* stats, float softmax_scale, const cva::DropParams& drop,
                   void* stream) {
  cva::BwdParams bp;
  bp.q = q;
  bp.k = k_rm;
  bp.v = v_rm;
  bp.o = o;
  bp.lse = lse;
  bp.dout = dout;
  bp.dq = dq;
  bp.dk = dk_rm;
  bp.dv = dv_rm;
  bp.delta = stats;
  bp.lse2 = stats + (size_t)p->T_loc * p->hq;
  bp.t = tables(*p);
  bp.n_dq_tiles = p->dq.n_tiles();
  bp.n_kv_tiles = p->dkdv.n_tiles();
  bp.n_zero_ranges = (int32_t)(p->zero_rows.size() / 2);
  bp.dq_heads_per_tile = p->fwd_heads_per_tile;
  bp.dq_head_groups = p->hq / p->fwd_heads_per_tile;
  bp.hq = p->hq;
  bp.hkv = p->hkv;
  bp.group = p->hq / p->hkv;
  bp.t_loc = (int32_t)p->T_loc;
  bp.t_total = p->T;
  bp.scale = softmax_scale;
  bp.scale_log2 = softmax_scale * 1.4426950408889634f;
  bp.drop = drop;
  hipError_t e = cva::launch_bwd(p->dtype, p->d_qk, p->d_v, bp, (hipStream_t)stream, hook());
  if (e != hipSuccess) return hip_fail(e, "backward launch");
  return CVA_OK;
}

}  // namespace

cva_status cva_bwd(const cva_plan* plan, const void* q, const void* k_rm, const void* v_rm,
                   const void* o, const float* lse, const void* dout, void* dq, void* dk_rm,
                   void* dv_rm, void* workspace, size_t ws_bytes, float softmax_scale,
                   void* stream) {
  const Plan* p = reinterpret_cast<const Plan*>(plan);
  cva_status st = check_bwd_args(p, q, k_rm, v_rm, o, lse, dout, dq, dk_rm, dv_rm, softmax_scale);
  if (st != CVA_OK) return st;
  const size_t need = cva_bwd_workspace_bytes(plan);
  if (workspace == nullptr || ws_bytes < need) {
    std::ostringstream os;
    os << "workspace needs " << need << " bytes";
    return fail(CVA_E_WORKSPACE, os.str());
  }
  return run_bwd(p, q, k_rm, v_rm, o, lse, dout, dq, dk_rm, dv_rm, (float*)workspace,
                 softmax_scale, kNoDrop, stream);
}

cva_status cva_bwd_dropout(const cva_plan* plan, const void* q, const void* k_rm, const void* v_rm,
                           const void* o, const float* lse, const void* dout, void* dq, void* dk_rm,
                           void* dv_rm, void* workspace, size_t ws_bytes, float softmax_scale,
                           float dropout_p, uint64_t seed, void* stream) {
  const Plan* p = reinterpret_cast<const Plan*>(plan);
  cva::DropParams d;
  cva_status st = make_drop(dropout_p, seed, &d);
  if (st != CVA_OK) return st;
  if ((st = check_bwd_args(p, q, k_rm, v_rm, o, lse, dout, dq, dk_rm, dv_rm, softmax_scale)) != CVA_OK) return st;
  const size_t need = cva_bwd_workspace_bytes(plan);
  if (workspace == nullptr || ws_bytes < need) {
    std::ostringstream os;
    os << "workspace needs " << need << " bytes";
    return fail(CVA_E_WORKSPACE, os.str());
  }
  return run_bwd(p, q, k_rm, v_rm, o, lse, dout, dq, dk_rm, dv_rm, (float*)workspace,
                 softmax_scale, d, stream);
}

size_t cva_bwd_noalloc_max_bytes(void) { return cva::kBwdNoAllocScratchBytes; }

cva_status cva_bwd_noalloc(const cva_plan* plan, const void* q, const void* k_rm,
                           const void* v_rm, const void* o, const float* lse, const void* dout,
                           void* dq, void* dk_rm, void* dv_rm, float softmax_scale, void* stream) {
  const Plan* p = reinterpret_cast<const Plan*>(plan);
  cva_status st = check_bwd_args(p, q, k_rm, v_rm, o, lse, dout, dq, dk_rm, dv_rm, softmax_scale);
  if (st != CVA_OK) return st;
  const size_t need = cva_bwd_workspace_bytes(plan);
  if (need > cva::kBwdNoAllocScratchBytes) {
    std::ostringstream os;
    os << "cva_bwd_noalloc holds at most " << cva::kBwdNoAllocScratchBytes
       << " bytes of row statistics; this plan needs " << need << " (use cva_bwd with a workspace)";
    return fail(CVA_E_WORKSPACE, os.str());
  }
  float* stats = nullptr;
  hipError_t e = cva::bwd_noalloc_scratch((hipStream_t)stream, &stats);
  if (e != hipSuccess) return hip_fail(e, "library device array (hipGetSymbolAddress)");
  return run_bwd(p, q, k_rm, v_rm, o, lse, dout, dq, dk_rm, dv_rm, stats, softmax_scale, kNoDrop, stream);
}

cva_status cva_plan_get_schedule(const cva_plan* plan, int32_t which, cva_schedule* out) {
  const Plan* p = reinterpret_cast<const Plan*>(plan);
  if (p == nullptr || out == nullptr) return fail(CVA_E_ARG, "plan or out is NULL");
  const cva::Schedule* s = which == 0   ? &p->fwd
                           : which == 1 ? &p->dq
                           : which == 2 ? &p->dkdv
                           : which == 3 ? &p->fwds
                                        : nullptr;
  if (s == nullptr) return fail(CVA_E_ARG, "which must be 0, 1, 2 or 3");
  out->tile_q = s->tile_q;
  out->tile_kv = s->tile_kv;
  out->n_tiles = s->n_tiles();
  out->n_spans = s->n_spans();
  out->tiles = s->tiles.data();
  out->spans = s->spans.data();
  return CVA_OK;
}

cva_status cva_plan_get_tables(const cva_plan* plan, cva_plan_tables* out) {
  const Plan* p = reinterpret_cast<const Plan*>(plan);
  if (p == nullptr || out == nullptr) return fail(CVA_E_ARG, "plan or out is NULL");
  out->n_segs = (int32_t)(p->segs.size() / cva::SEG_INTS);
  out->segs = p->segs.data();
  out->kv_index_len = (int64_t)p->kv_index.size();
  out->kv_index = p->kv_index.data();
  out->n_rows = (int64_t)(p->row_iv.size() / 4);
  out->row_iv = p->row_iv.data();
  out->n_zero_ranges = (int32_t)(p->zero_rows.size() / 2);
  out->zero_rows = p->zero_rows.data();
  out->n_split_items = (int32_t)p->fwds_slot.size();
  out->split_slot = p->fwds_slot.data();
  out->n_combine = (int32_t)(p->fwds_combine.size() / cva::CB_INTS);
  out->split_combine = p->fwds_combine.data();
  out->n_split_slots = p->n_split_slots;
  out->fwd_deal_wgs = p->fwd_deal.wgs;
  out->fwd_deal_start = p->fwd_deal.start.data();
  out->fwd_deal_items = p->fwd_deal.items.data();
  out->n_fwd_deal_items = (int32_t)p->fwd_deal.items.size();
  out->split_deal_wgs = p->fwds_deal.wgs;
  out->split_deal_start = p->fwds_deal.start.data();
  out->split_deal_items = p->fwds_deal.items.data();
  out->n_split_deal_items = (int32_t)p->fwds_deal.items.size();
  return CVA_OK;
}

cva_status cva_placement_create(const int32_t* cu_seqlens, int32_t n_seqs, const cva_mask_desc* mask,
                                int32_t n_devices, int32_t block, int32_t hq, int32_t hkv,
                                int32_t d_qk, int32_t d_v, int32_t dtype, double epsilon,
                                cva_placement** out) {
  if (out == nullptr) return fail(CVA_E_ARG, "out is NULL");
  *out = nullptr;
  if (cu_seqlens == nullptr) return fail(CVA_E_ARG, "cu_seqlens is NULL");
  if (n_seqs < 1) return fail(CVA_E_CU_SEQLENS, "cu_seqlens must hold at least one sub-sequence");
  if (cu_seqlens[0] != 0) return fail(CVA_E_CU_SEQLENS, "cu_seqlens must start at 0");
  for (int32_t i = 0; i < n_seqs; ++i)
    if (cu_seqlens[i + 1] <= cu_seqlens[i]) return fail(CVA_E_CU_SEQLENS, "cu_seqlens must be strictly increasing");
  if (n_devices < 1 || n_devices > 64) return fail(CVA_E_RANK, "n_devices must be in [1, 64]");
  if (!(epsilon >= 0.0) || epsilon > 1e6) return fail(CVA_E_ARG, "epsilon must be >= 0");
  if (block < 1) return fail(CVA_E_ARG, "block must be >= 1");
  if (hq < 1 || hkv < 1 || d_qk < 1 || d_v < 1) return fail(CVA_E_HEADS, "head counts and dims must be >= 1");
  if (dtype != CVA_BF16 && dtype != CVA_FP16 && dtype != CVA_FP32) return fail(CVA_E_DTYPE, "unknown dtype");
  cva_status st = cva::validate_mask(mask, cu_seqlens, n_seqs);
  if (st != CVA_OK) return st;
  auto* pl = new (std::nothrow) cva::Placement();
  if (pl == nullptr) return fail(CVA_E_ARG, "out of host memory");
  try {
    Plan& m = pl->mask;
    m.n_seqs = n_seqs;
    m.cu.assign(cu_seqlens, cu_seqlens + n_seqs + 1);
    if (mask != nullptr) {
      m.mask_type = mask->type;
      m.sink = mask->sink;
      m.window = mask->window;
      if (mask->type == CVA_MASK_BLOCKWISE) m.block = mask->block;
      if (mask->type == CVA_MASK_SHARED_PREFIX) {
        m.n_branches = mask->n_branches;
        m.branch_bounds.assign(mask->branch_bounds, mask->branch_bounds + (size_t)n_seqs * (mask->n_branches + 1));
      }
    }
    pl->n_devices = n_devices;
    pl->block = block;
    pl->hq = hq;
    pl->hkv = hkv;
    pl->d_qk = d_qk;
    pl->d_v = d_v;
    pl->dtype = dtype;
    pl->epsilon = epsilon;
    st = cva::build_placement(*pl);
  } catch (const std::bad_alloc&) {
    st = fail(CVA_E_ARG, "out of host memory while placing blocks");
  }
  if (st != CVA_OK) {
    delete pl;
    return st;
  }
  *out = reinterpret_cast<cva_placement*>(pl);
  return CVA_OK;
}

cva_status cva_placement_get(const cva_placement* placement, cva_placement_info* out) {
  const auto* pl = reinterpret_cast<const cva::Placement*>(placement);
  if (pl == nullptr || out == nullptr) return fail(CVA_E_ARG, "placement or out is NULL");
  out->n_devices = pl->n_devices;
  out->block = pl->block;
  out->n_data_blocks = (int32_t)(pl->data.size() / 4);
  out->n_comp_blocks = (int32_t)pl->comp_pairs.size();
  out->data_blocks = pl->data.data();
  out->comp_blocks = pl->comp.data();
  out->comp_pairs = pl->comp_pairs.data();
  out->device_tokens = pl->device_tokens.data();
  out->device_pairs = pl->device_pairs.data();
  out->device_send_bytes = pl->device_send_bytes.data();
  out->device_recv_bytes = pl->device_recv_bytes.data();
  out->total_comm_bytes = pl->total_comm_bytes;
  out->block_comm_bytes = pl->block_comm_bytes;
  out->zigzag_valid = pl->zigzag_ok ? 1 : 0;
  out->zigzag_pairs = pl->zigzag_pairs.data();
  out->zigzag_comm_bytes = pl->zigzag_comm_bytes;
  return CVA_OK;
}

cva_status cva_placement_plan_create(const cva_placement* placement, int32_t device,
                                     cva_plan** out) {
  cva::set_error("");
  if (out == nullptr) return fail(CVA_E_ARG, "out is NULL");
  *out = nullptr;
  const auto* pl = reinterpret_cast<const cva::Placement*>(placement);
  if (pl == nullptr) return fail(CVA_E_ARG, "placement is NULL");
  Plan* p = new (std::nothrow) Plan();
  if (p == nullptr) return fail(CVA_E_ARG, "out of host memory");
  cva_status st;
  try {
    st = cva::build_placed_plan(*pl, device, *p);
  } catch (const std::bad_alloc&) {
    st = fail(CVA_E_ARG, "out of host memory while building the plan");
  }
  if (st != CVA_OK) {
    delete p;
    return st;
  }
  *out = reinterpret_cast<cva_plan*>(p);
  return CVA_OK;
}

void cva_placement_destroy(cva_placement* placement) {
  delete reinterpret_cast<cva::Placement*>(placement);
}

cva_status cva_timing_enable(int32_t on) {
  std::lock_guard<std::mutex> lock(g_timer.mu);
  if (on) {
    hipError_t e = g_timer.drain();
    g_timer.reset();
    g_timer.on = true;
    if (e != hipSuccess) return hip_fail(e, "timing drain");
  } else {
    g_timer.on = false;
  }
  return CVA_OK;
}

cva_status cva_timing_select(uint32_t kernel_mask) {
  std::lock_guard<std::mutex> lock(g_timer.mu);
  g_timer.mask = kernel_mask;
  return CVA_OK;
}

cva_status cva_timing_read(cva_kernel_times* out) {
  if (out == nullptr) return fail(CVA_E_ARG, "out is NULL");
  std::lock_guard<std::mutex> lock(g_timer.mu);
  hipError_t e = g_timer.drain();
  for (int k = 0; k < CVA_N_KERNELS; ++k) {
    out->launches[k] = g_timer.launches[k];
    out->total_ms[k] = g_timer.total_ms[k];
  }
  if (e != hipSuccess) return hip_fail(e, "timing events");
  return CVA_OK;
}

}  // extern "C"
