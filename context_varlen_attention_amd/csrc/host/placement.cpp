// Block placement over R devices (DCP paper, section 4.1 and its placement
// model): the attention of a batch is cut into data blocks (the Q, K/V and O
// rows of `block` consecutive tokens of one sequence, placed together, all
// heads) and computation blocks (one Q block against one K/V block of the same
// sequence, created only where the mask between them is not all zero).
//
// The page places blocks by balanced hypergraph partitioning: one hyperedge per
// data block joining it to every computation block that reads or writes it,
// computation weight balanced within a tolerance epsilon, data balanced as well
// as possible, and the connectivity sum_e size(e) * (spanned devices - 1), which
// is the bytes moved when a device fetches a remote block once and reuses it,
// minimised.  The solver it uses is a third-party multi-level partitioner; this
// is a greedy stand-in with the same constraints and objective:
//  1. data blocks go out in runs of consecutive blocks per device, up to the
//     per-device token target; two seeds are tried, plain runs in sequence
//     order and mirrored runs (block k of a sequence with n blocks on the
//     device the zig-zag split gives the 2R-slot position of k), which balance
//     causal rows;
//  2. computation blocks, heaviest first, go to the device, among those whose
//     visible-pair load stays within (1 + epsilon) of the mean, that adds the
//     least connectivity (a device already holding or fetching all three of
//     its data blocks adds none), ties to the less loaded device, or to the
//     least loaded device when none fits;
// and the seed with the lower maximum load, then the lower connectivity, wins.
// It is host work only: the kernels of this library compute one rank's share
// under the RFC's zig-zag split, which is reported beside the placement.
#include <algorithm>
#include <numeric>

#include "plan.hpp"

namespace cva {

namespace {

struct Sizes {
  int64_t q_row, kv_row, o_row;
};

// Result of one seed: device of every data block and computation block.
struct Assign {
  std::vector<int32_t> data_dev, comp_dev;
  std::vector<int64_t> pairs;
  int64_t max_pairs = 0, connectivity = 0;
};

// Pass 2 for fixed data devices.
void place_computation(const Placement& pl, const std::vector<int32_t>& first_block, const Sizes& sz,
                       const std::vector<int32_t>& order, int64_t total_pairs, Assign& a) {
  const int32_t R = pl.n_devices;
  const int32_t n_data = (int32_t)a.data_dev.size();
  // span masks of the Q/O hyperedges (same computation blocks) and the K/V hyperedges
  std::vector<uint64_t> span_q(n_data), span_kv(n_data);
  for (int32_t d = 0; d < n_data; ++d) span_q[d] = span_kv[d] = uint64_t(1) << a.data_dev[d];
  a.pairs.assign(R, 0);
  a.comp_dev.assign(pl.comp_pairs.size(), -1);
  const double cap = (double)total_pairs / R * (1.0 + pl.epsilon);
  for (int32_t c : order) {
    const int32_t seq = pl.comp[(size_t)c * 4], qb = pl.comp[(size_t)c * 4 + 1], kb = pl.comp[(size_t)c * 4 + 2];
    const int32_t dq = first_block[seq] + qb, dk = first_block[seq] + kb;
    const int64_t qtok = pl.data[(size_t)dq * 4 + 2], ktok = pl.data[(size_t)dk * 4 + 2];
    auto added = [&](int32_t dev) {
      const uint64_t bit = uint64_t(1) << dev;
      int64_t v = 0;
      if (!(span_q[dq] & bit)) v += qtok * (sz.q_row + sz.o_row);
      if (!(span_kv[dk] & bit)) v += ktok * sz.kv_row;
      return v;
    };
    int32_t best = -1;
    int64_t best_v = 0;
    for (int32_t dev = 0; dev < R; ++dev) {
      if ((double)(a.pairs[dev] + pl.comp_pairs[c]) > cap) continue;
      const int64_t v = added(dev);
      if (best < 0 || v < best_v || (v == best_v && a.pairs[dev] < a.pairs[best])) {
        best = dev;
        best_v = v;
      }
    }
    if (best < 0) {
      best = (int32_t)(std::min_element(a.pairs.begin(), a.pairs.end()) - a.pairs.begin());
      best_v = added(best);
    }
    a.comp_dev[c] = best;
    a.pairs[best] += pl.comp_pairs[c];
    a.connectivity += best_v;
    span_q[dq] |= uint64_t(1) << best;
    span_kv[dk] |= uint64_t(1) << best;
  }
  a.max_pairs = *std::max_element(a.pairs.begin(), a.pairs.end());
}

}  // namespace

cva_status build_placement(Placement& pl) {
  const Plan& m = pl.mask;  // mask fields and cu only
  const int32_t B = pl.block, R = pl.n_devices;
  const int32_t esz = pl.dtype == CVA_FP32 ? 4 : 2;
  Sizes sz;
  sz.q_row = (int64_t)pl.hq * pl.d_qk * esz;
  sz.o_row = (int64_t)pl.hq * pl.d_v * esz;
  sz.kv_row = (int64_t)pl.hkv * (pl.d_qk + pl.d_v) * esz;

  // ---- data blocks and computation blocks (visible pairs per head) ----
  pl.data.clear();
  pl.comp.clear();
  pl.comp_pairs.clear();
  std::vector<int32_t> first_block(m.n_seqs + 1, 0);
  for (int32_t i = 0; i < m.n_seqs; ++i) {
    const int32_t L = m.cu[i + 1] - m.cu[i];
    first_block[i] = (int32_t)(pl.data.size() / 4);
    for (int32_t t0 = 0; t0 < L; t0 += B) pl.data.insert(pl.data.end(), {i, t0, std::min(B, L - t0), -1});
    const int32_t nb = (L + B - 1) / B;
    std::vector<int64_t> cnt((size_t)nb, 0);
    for (int32_t qb = 0; qb < nb; ++qb) {
      std::fill(cnt.begin(), cnt.end(), 0);
      for (int32_t q = qb * B; q < std::min(L, (qb + 1) * B); ++q) {
        int32_t iv[4];
        position_intervals(m, i, q, iv);
        const KeySet rs = key_set(iv);
        for (int k = 0; k < rs.n; ++k) {
          int32_t a = rs.v[k].first;
          const int32_t e = rs.v[k].second;
          while (a < e) {  // split the interval at block boundaries
            const int32_t kb = a / B;
            const int32_t end = std::min(e, (kb + 1) * B);
            cnt[kb] += end - a;
            a = end;
          }
        }
      }
      for (int32_t kb = 0; kb < nb; ++kb)
        if (cnt[kb] > 0) {
          pl.comp.insert(pl.comp.end(), {i, qb, kb, -1});
          pl.comp_pairs.push_back(cnt[kb]);
        }
    }
  }
  first_block[m.n_seqs] = (int32_t)(pl.data.size() / 4);
  const int32_t n_data = (int32_t)(pl.data.size() / 4);
  const int32_t n_comp = (int32_t)pl.comp_pairs.size();
  const int64_t total_tokens = m.cu[m.n_seqs];
  const int64_t total_pairs = std::accumulate(pl.comp_pairs.begin(), pl.comp_pairs.end(), (int64_t)0);

  std::vector<int32_t> order(n_comp);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(),
                   [&](int32_t a, int32_t b) { return pl.comp_pairs[a] > pl.comp_pairs[b]; });

  // ---- pass 1 (two seeds) + pass 2 ----
  const double tok_target = (double)total_tokens / R;
  Assign best;
  for (int seed = 0; seed < 2; ++seed) {
    Assign a;
    a.data_dev.assign(n_data, -1);
    std::vector<int64_t> tokens(R, 0);
    for (int32_t i = 0; i < m.n_seqs; ++i) {
      const int32_t nb = first_block[i + 1] - first_block[i];
      int32_t prev = -1;
      for (int32_t k = 0; k < nb; ++k) {
        int32_t want = prev;
        if (seed == 1) {  // mirrored runs: the zig-zag slot (of 2R) holding the block's middle
          const int32_t slot = (int32_t)(((2 * (int64_t)k + 1) * R) / nb);
          want = slot < R ? slot : 2 * R - 1 - slot;
        }
        const int32_t d = first_block[i] + k;
        const int32_t tok = pl.data[(size_t)d * 4 + 2];
        int32_t dev = want;
        if (dev < 0 || (double)(tokens[dev] + tok) > tok_target + 0.5)
          dev = (int32_t)(std::min_element(tokens.begin(), tokens.end()) - tokens.begin());
        a.data_dev[d] = dev;
        tokens[dev] += tok;
        prev = dev;
      }
    }
    place_computation(pl, first_block, sz, order, total_pairs, a);
    if (seed == 0 || a.max_pairs < best.max_pairs ||
        (a.max_pairs == best.max_pairs && a.connectivity < best.connectivity))
      best = std::move(a);
  }

  // ---- write the winner and its accounting ----
  pl.device_tokens.assign(R, 0);
  pl.device_pairs = best.pairs;
  pl.device_send_bytes.assign(R, 0);
  pl.device_recv_bytes.assign(R, 0);
  for (int32_t d = 0; d < n_data; ++d) {
    pl.data[(size_t)d * 4 + 3] = best.data_dev[d];
    pl.device_tokens[best.data_dev[d]] += pl.data[(size_t)d * 4 + 2];
  }
  pl.block_comm_bytes = 0;
  std::vector<uint64_t> span_q(n_data), span_kv(n_data);
  for (int32_t d = 0; d < n_data; ++d) span_q[d] = span_kv[d] = uint64_t(1) << best.data_dev[d];
  for (int32_t c = 0; c < n_comp; ++c) {
    const int32_t dev = best.comp_dev[c];
    pl.comp[(size_t)c * 4 + 3] = dev;
    const int32_t seq = pl.comp[(size_t)c * 4], dq = first_block[seq] + pl.comp[(size_t)c * 4 + 1],
                  dk = first_block[seq] + pl.comp[(size_t)c * 4 + 2];
    const int64_t qtok = pl.data[(size_t)dq * 4 + 2], ktok = pl.data[(size_t)dk * 4 + 2];
    if (best.data_dev[dq] != dev) pl.block_comm_bytes += qtok * (sz.q_row + sz.o_row);
    if (best.data_dev[dk] != dev) pl.block_comm_bytes += ktok * sz.kv_row;
    span_q[dq] |= uint64_t(1) << dev;
    span_kv[dk] |= uint64_t(1) << dev;
  }
  // connectivity: inputs leave their owner once per computing device, partial
  // outputs come back to the owner of the Q block once per computing device
  pl.total_comm_bytes = 0;
  for (int32_t d = 0; d < n_data; ++d) {
    const int32_t home = best.data_dev[d];
    const int64_t tok = pl.data[(size_t)d * 4 + 2];
    for (int32_t dev = 0; dev < R; ++dev) {
      if (dev == home) continue;
      if (span_q[d] & (uint64_t(1) << dev)) {
        pl.device_send_bytes[home] += tok * sz.q_row;
        pl.device_recv_bytes[dev] += tok * sz.q_row;
        pl.device_send_bytes[dev] += tok * sz.o_row;
        pl.device_recv_bytes[home] += tok * sz.o_row;
        pl.total_comm_bytes += tok * (sz.q_row + sz.o_row);
      }
      if (span_kv[d] & (uint64_t(1) << dev)) {
        pl.device_send_bytes[home] += tok * sz.kv_row;
        pl.device_recv_bytes[dev] += tok * sz.kv_row;
        pl.total_comm_bytes += tok * sz.kv_row;
      }
    }
  }

  // ---- the RFC's zig-zag split for comparison ----
  pl.zigzag_pairs.assign(R, 0);
  pl.zigzag_ok = true;
  for (int32_t i = 0; i < m.n_seqs && pl.zigzag_ok; ++i)
    if ((m.cu[i + 1] - m.cu[i]) % (2 * R) != 0) pl.zigzag_ok = false;
  if (pl.zigzag_ok) {
    for (int32_t i = 0; i < m.n_seqs; ++i) {
      const int32_t c = (m.cu[i + 1] - m.cu[i]) / (2 * R);
      for (int32_t s = 0; s < R; ++s)
        for (int32_t j : {s, 2 * R - 1 - s})
          for (int32_t q = j * c; q < (j + 1) * c; ++q) {
            int32_t iv[4];
            position_intervals(m, i, q, iv);
            const KeySet rs = key_set(iv);
            for (int k = 0; k < rs.n; ++k) pl.zigzag_pairs[s] += rs.v[k].second - rs.v[k].first;
          }
    }
  }
  // every rank gathers the K/V rows of all other ranks
  pl.zigzag_comm_bytes = (int64_t)(R - 1) * total_tokens * sz.kv_row;
  return CVA_OK;
}

}  // namespace cva

namespace cva {

// One device's share of a placement as a plan.  The packed batch is addressed
// as it is (row = packed token), so every device reads its local and fetched
// blocks in place: segments are the Q blocks the device computes on (all of
// their sequence's keys addressable, in-sequence positions), and each
// computation block becomes forward items restricted to its K/V block's keys
// (DCP paper, section 4.1: a computation block pairs one Q block with one K/V
// block; Fig. 9(b): blocks that feed the same output block are reduced).
cva_status build_placed_plan(const Placement& pl, int32_t device, Plan& p) {
  const Plan& m = pl.mask;
  if (device < 0 || device >= pl.n_devices) {
    set_error("device must be in [0, n_devices)");
    return CVA_E_RANK;
  }
  if (pl.dtype != CVA_BF16 && pl.dtype != CVA_FP16) {
    set_error("a placement share runs on the bf16/fp16 kernels");
    return CVA_E_UNSUPPORTED;
  }
  if (pl.hq % pl.hkv != 0) {
    set_error("query heads must be a multiple of K/V heads");
    return CVA_E_HEADS;
  }
  if (!head_dims_supported(pl.dtype, pl.d_qk, pl.d_v)) {
    set_error("no kernel for these head dims; supported: (64,64), (128,128), (192,128)");
    return CVA_E_HEADDIM;
  }
  if (pl.block % kFwdTileKv != 0) {
    set_error("running a placement share needs a block size that is a multiple of 64 (the K/V tile)");
    return CVA_E_UNSUPPORTED;
  }
  const int32_t B = pl.block;
  p.n_seqs = m.n_seqs;
  p.cp_size = 1;
  p.rank = 0;
  p.hq = pl.hq;
  p.hkv = pl.hkv;
  p.d_qk = pl.d_qk;
  p.d_v = pl.d_v;
  p.dtype = pl.dtype;
  p.mask_type = m.mask_type;
  p.sink = m.sink;
  p.window = m.window;
  p.n_branches = m.n_branches;
  p.block = m.block;
  p.cu = m.cu;
  p.branch_bounds = m.branch_bounds;
  p.placed = true;
  p.placed_device = device;
  p.T = p.T_loc = m.cu[m.n_seqs];
  p.kv_index.resize((size_t)p.T);
  std::iota(p.kv_index.begin(), p.kv_index.end(), 0);  // one run per sequence, from its first token
  p.row_iv.assign((size_t)p.T * 4, 0);
  for (int32_t i = 0; i < m.n_seqs; ++i)
    for (int32_t q = 0; q < m.cu[i + 1] - m.cu[i]; ++q)
      position_intervals(p, i, q, &p.row_iv[((size_t)m.cu[i] + q) * 4]);
  // the device's computation blocks in (sequence, Q block, K/V block) order
  std::vector<int32_t> mine;
  for (int32_t c = 0; c < (int32_t)pl.comp_pairs.size(); ++c)
    if (pl.comp[(size_t)c * 4 + 3] == device) mine.push_back(c);
  std::sort(mine.begin(), mine.end(), [&](int32_t a, int32_t b) {
    for (int f = 0; f < 3; ++f)
      if (pl.comp[(size_t)a * 4 + f] != pl.comp[(size_t)b * 4 + f])
        return pl.comp[(size_t)a * 4 + f] < pl.comp[(size_t)b * 4 + f];
    return false;
  });
  std::vector<PlacedBlock> blocks;
  p.segs.clear();
  p.visible_pairs = 0;
  int32_t last_seq = -1, last_qb = -1;
  for (int32_t c : mine) {
    const int32_t seq = pl.comp[(size_t)c * 4], qb = pl.comp[(size_t)c * 4 + 1], kb = pl.comp[(size_t)c * 4 + 2];
    const int32_t L = m.cu[seq + 1] - m.cu[seq];
    if (seq != last_seq || qb != last_qb) {
      p.segs.insert(p.segs.end(), {seq, qb, std::min(B, L - qb * B), L, m.cu[seq] + qb * B, m.cu[seq],
                                   qb * B, L});
      last_seq = seq;
      last_qb = qb;
    }
    blocks.push_back({(int32_t)(p.segs.size() / SEG_INTS) - 1, kb * B, std::min(L, (kb + 1) * B)});
    p.visible_pairs += pl.comp_pairs[c];
  }
  p.visible_pairs_per_rank.assign(1, p.visible_pairs);
  cva_status st = build_placed_schedule(p, blocks);
  if (st != CVA_OK) return st;
  build_blob(p);
  return CVA_OK;
}

}  // namespace cva
