// Block-mask tile scheduler.
//
// DCP paper (block-wise attention and its computation blocks): a computation
// block pairs a Q block with a K/V block and is only created where the mask
// between them is not all zero, so masked work is discarded before it is
// launched.  This file does that on kernel tiles.
//
// Every query row's visible keys form at most two intervals of in-sequence
// positions (row_intervals): causal [0, q]; lambda [0, min(sink, q+1)) and
// [q-window+1, q] (DCP Fig. 6(b)); causal blockwise [0, sink blocks) and the
// window of blocks ending with the query's block, the last block causal
// (DCP Fig. 6(c)); shared prefix [0, q] inside the question,
// else [0, prefix) and [answer start, q] (DCP Fig. 6(d)).  For a tile of
// query rows the union U of its rows' sets says which K/V tiles are non-empty
// and the intersection F which are full (no element-wise mask needed); tiles
// in U but not inside F are partial.  Tiles are emitted as spans of equal
// status, so the cost is linear in the number of spans, not in the mask area.
//
// Launch order puts the tiles with the most work first (longest-processing-
// time order) so that long causal rows do not trail at the end of a launch.
#include <algorithm>
#include <array>
#include <atomic>
#include <cstdlib>
#include <cstring>
#include <new>
#include <numeric>
#include <thread>
#include <utility>

#include "plan.hpp"

namespace cva {

namespace {

using Iv = std::pair<int32_t, int32_t>;  // [first, end)
using IvList = std::vector<Iv>;

// A row's visible set: at most two disjoint, sorted intervals.
using RowSet = KeySet;
inline RowSet row_set(const int32_t* iv) { return key_set(iv); }

// Intersection of a sorted disjoint list with a row set, in place.
void intersect_into(IvList& F, const RowSet& s, IvList& tmp) {
  tmp.clear();
  size_t i = 0;
  int j = 0;
  while (i < F.size() && j < s.n) {
    const int32_t lo = std::max(F[i].first, s.v[j].first);
    const int32_t hi = std::min(F[i].second, s.v[j].second);
    if (hi > lo) tmp.push_back({lo, hi});
    if (F[i].second < s.v[j].second) ++i; else ++j;
  }
  F.swap(tmp);
}

struct SpanOut {
  int32_t t0, t1, partial;
};

// Scratch buffers reused across tiles so the hot loop does not allocate.
struct Scratch {
  IvList all, U, F, tmp, ne, full;
  std::vector<SpanOut> spans;
};

// Spans of tiles of width `bn` given the union U and intersection F of the rows' visible sets.
void tile_spans(Scratch& w, int32_t bn) {
  w.ne.clear();
  for (const Iv& u : w.U) {
    const int32_t t0 = u.first / bn, t1 = (u.second + bn - 1) / bn;
    if (!w.ne.empty() && t0 <= w.ne.back().second)
      w.ne.back().second = std::max(w.ne.back().second, t1);
    else
      w.ne.push_back({t0, t1});
  }
  w.full.clear();
  for (const Iv& f : w.F) {
    const int32_t t0 = (f.first + bn - 1) / bn, t1 = f.second / bn;
    if (t1 > t0) w.full.push_back({t0, t1});
  }
  w.spans.clear();
  size_t k = 0;
  for (const Iv& r : w.ne) {
    int32_t cur = r.first;
    while (k < w.full.size() && w.full[k].second <= cur) ++k;
    while (k < w.full.size() && w.full[k].first < r.second) {
      const int32_t f0 = std::max(w.full[k].first, cur), f1 = std::min(w.full[k].second, r.second);
      if (f0 > cur) w.spans.push_back({cur, f0, 1});
      if (f1 > f0) w.spans.push_back({f0, f1, 0});
      cur = std::max(cur, f1);
      if (w.full[k].second <= r.second) ++k; else break;
    }
    if (cur < r.second) w.spans.push_back({cur, r.second, 1});
  }
}

// Union U and intersection F of the visible sets of rows [a0, a1) of a segment.
void tile_sets(const Plan& p, int seg, int32_t a0, int32_t a1, Scratch& w) {
  const int32_t row0 = p.segs[(size_t)seg * SEG_INTS + SEG_QROW0];
  w.all.clear();
  w.F.clear();
  bool monotone = true;  // row starts/ends non-decreasing: union is a sweep, no sort
  for (int32_t a = a0; a < a1; ++a) {
    const RowSet s = row_set(&p.row_iv[(size_t)(row0 + a) * 4]);
    for (int k = 0; k < s.n; ++k) {
      if (!w.all.empty() && s.v[k].first < w.all.back().first) monotone = false;
      w.all.push_back(s.v[k]);
    }
    if (a == a0) {
      for (int k = 0; k < s.n; ++k) w.F.push_back(s.v[k]);
    } else if (!w.F.empty()) {
      intersect_into(w.F, s, w.tmp);
    }
  }
  if (!monotone) std::sort(w.all.begin(), w.all.end());
  w.U.clear();
  for (const Iv& x : w.all) {
    if (!w.U.empty() && x.first <= w.U.back().second)
      w.U.back().second = std::max(w.U.back().second, x.second);
    else
      w.U.push_back(x);
  }
}

// Runs f(i) for i in [0, n) on up to kPlanThreads host threads when the batch is
// large (rows >= kPlanParallelRows), else inline; every i writes only its own
// outputs, so the result does not depend on the thread count.  CVA_PLAN_THREADS
// in the environment lowers the cap (1: always inline).
constexpr int32_t kPlanThreads = 8;
constexpr int64_t kPlanParallelRows = 32768;
template <typename Fn>
void parallel_for(int32_t n, int64_t rows, Fn f) {
  int32_t cap = kPlanThreads;
  if (const char* v = std::getenv("CVA_PLAN_THREADS")) cap = std::max(1, std::min(kPlanThreads, std::atoi(v)));
  const int32_t hw = (int32_t)std::max(1u, std::thread::hardware_concurrency());
  const int32_t nt = rows >= kPlanParallelRows ? std::min({hw, cap, n}) : 1;
  if (nt <= 1) {
    for (int32_t i = 0; i < n; ++i) f(i);
    return;
  }
  std::atomic<int32_t> next{0};
  std::atomic<bool> failed{false};
  std::vector<std::thread> th;
  th.reserve(nt);
  for (int32_t t = 0; t < nt; ++t)
    th.emplace_back([&]() {
      try {
        for (int32_t i = next++; i < n && !failed; i = next++) f(i);
      } catch (...) {  // out of memory in a worker: reported by the caller's thread
        failed = true;
      }
    });
  for (auto& x : th) x.join();
  if (failed) throw std::bad_alloc();
}

// Intersection of two sorted disjoint interval lists, into F.
void intersect_lists(IvList& F, const Iv* g, int32_t ng, IvList& tmp) {
  tmp.clear();
  size_t i = 0;
  int32_t j = 0;
  while (i < F.size() && j < ng) {
    const int32_t lo = std::max(F[i].first, g[j].first);
    const int32_t hi = std::min(F[i].second, g[j].second);
    if (hi > lo) tmp.push_back({lo, hi});
    if (F[i].second < g[j].second) ++i; else ++j;
  }
  F.swap(tmp);
}

// Union and intersection of the visible sets of every kBlockRows-row block of
// every segment, computed once; the sets of a Q tile (a whole number of blocks
// from the segment's start) are then merged from its blocks instead of being
// recomputed row by row for each schedule.
constexpr int32_t kBlockRows = 32;
struct BlockSets {
  std::vector<int32_t> seg_block0;  // [nseg + 1] first block of each segment
  std::vector<int32_t> u_off, f_off;  // [nblocks + 1] offsets into U / F
  IvList U, F;
  void build(const Plan& p) {
    const int32_t nseg = (int32_t)(p.segs.size() / SEG_INTS);
    seg_block0.assign(nseg + 1, 0);
    std::vector<std::pair<int32_t, int32_t>> blocks;  // (segment, first row)
    for (int32_t sg = 0; sg < nseg; ++sg) {
      const int32_t q_len = p.segs[sg * SEG_INTS + SEG_QLEN];
      for (int32_t a0 = 0; a0 < q_len; a0 += kBlockRows) blocks.push_back({sg, a0});
      seg_block0[sg + 1] = (int32_t)blocks.size();
    }
    // chunks of blocks (in parallel for large batches), concatenated in order
    constexpr int32_t kChunk = 64;
    const int32_t nb = (int32_t)blocks.size(), nchunk = (nb + kChunk - 1) / kChunk;
    struct Part {
      IvList U, F;
      std::vector<int32_t> un, fn;  // intervals per block
    };
    std::vector<Part> parts(nchunk);
    parallel_for(nchunk, p.T_loc, [&](int32_t c) {
      Part& pt = parts[c];
      Scratch w;
      for (int32_t b = c * kChunk; b < std::min(nb, (c + 1) * kChunk); ++b) {
        const int32_t sg = blocks[b].first, a0 = blocks[b].second;
        const int32_t q_len = p.segs[sg * SEG_INTS + SEG_QLEN];
        tile_sets(p, sg, a0, std::min(q_len, a0 + kBlockRows), w);
        pt.U.insert(pt.U.end(), w.U.begin(), w.U.end());
        pt.F.insert(pt.F.end(), w.F.begin(), w.F.end());
        pt.un.push_back((int32_t)w.U.size());
        pt.fn.push_back((int32_t)w.F.size());
      }
    });
    u_off.assign(1, 0);
    f_off.assign(1, 0);
    U.clear();
    F.clear();
    for (const Part& pt : parts) {
      U.insert(U.end(), pt.U.begin(), pt.U.end());
      F.insert(F.end(), pt.F.begin(), pt.F.end());
      for (size_t b = 0; b < pt.un.size(); ++b) {
        u_off.push_back(u_off.back() + pt.un[b]);
        f_off.push_back(f_off.back() + pt.fn[b]);
      }
    }
  }
  // w.U / w.F of rows [a0, a1) of segment sg (a0 a multiple of kBlockRows)
  void tile(int32_t sg, int32_t a0, int32_t a1, Scratch& w) const {
    const int32_t b0 = seg_block0[sg] + a0 / kBlockRows;
    const int32_t b1 = seg_block0[sg] + (a1 + kBlockRows - 1) / kBlockRows;
    w.all.clear();
    bool monotone = true;
    for (int32_t b = b0; b < b1; ++b)
      for (int32_t k = u_off[b]; k < u_off[b + 1]; ++k) {
        if (!w.all.empty() && U[k].first < w.all.back().first) monotone = false;
        w.all.push_back(U[k]);
      }
    if (!monotone) std::sort(w.all.begin(), w.all.end());
    w.U.clear();
    for (const Iv& x : w.all) {
      if (!w.U.empty() && x.first <= w.U.back().second)
        w.U.back().second = std::max(w.U.back().second, x.second);
      else
        w.U.push_back(x);
    }
    w.F.assign(F.begin() + f_off[b0], F.begin() + f_off[b0 + 1]);
    for (int32_t b = b0 + 1; b < b1 && !w.F.empty(); ++b)
      intersect_lists(w.F, F.data() + f_off[b], f_off[b + 1] - f_off[b], w.tmp);
  }
};

// First cut of a segment's Q tiles.  Under the causal blockwise mask the tiles
// are cut at in-sequence positions that are multiples of tile_q (so the first
// tile may be short): a segment that starts inside a mask block would otherwise
// have every tile straddle a block boundary and walk the K/V tiles of one more
// block (on an 8-sequence batch with blocks of 256 tokens this cuts the
// forward's K/V tile steps by 12 %).  Cuts stay multiples of the 32-row blocks
// the visible sets are built from; other masks cut from the segment's start.
int32_t first_cut(const Plan& p, int32_t sg, int32_t tile_q) {
  if (p.mask_type != CVA_MASK_BLOCKWISE) return tile_q;
  const int32_t q_len = p.segs[sg * SEG_INTS + SEG_QLEN];
  const int32_t qpos0 = p.segs[sg * SEG_INTS + SEG_QPOS0];
  const int32_t f = ((tile_q - qpos0 % tile_q) % tile_q) & ~(kBlockRows - 1);
  return f > 0 && f < q_len ? f : tile_q;
}

void build_q_schedule(const Plan& p, const BlockSets& bs, Schedule& s, int32_t tile_q, int32_t tile_kv) {
  s.tile_q = tile_q;
  s.tile_kv = tile_kv;
  s.tiles.clear();
  s.spans.clear();
  s.tile_pairs = 0;
  struct Rec { int32_t seg, q0, rows, span0, nspan; int64_t cost; };
  std::vector<Rec> recs;
  std::vector<SpanOut> all_spans;
  Scratch w;
  const int32_t nseg = (int32_t)(p.segs.size() / SEG_INTS);
  for (int32_t sg = 0; sg < nseg; ++sg) {
    const int32_t q_len = p.segs[sg * SEG_INTS + SEG_QLEN];
    for (int32_t a0 = 0, a1 = std::min(q_len, first_cut(p, sg, tile_q)); a0 < q_len;
         a0 = a1, a1 = std::min(q_len, a1 + tile_q)) {
      bs.tile(sg, a0, a1, w);
      tile_spans(w, tile_kv);
      Rec r{sg, a0, a1 - a0, (int32_t)all_spans.size(), (int32_t)w.spans.size(), 0};
      for (const SpanOut& x : w.spans) r.cost += x.t1 - x.t0;
      all_spans.insert(all_spans.end(), w.spans.begin(), w.spans.end());
      recs.push_back(r);
    }
  }
  std::vector<size_t> order(recs.size());
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(),
                   [&](size_t x, size_t y) { return recs[x].cost > recs[y].cost; });
  s.tiles.reserve(recs.size() * QT_INTS);
  s.spans.reserve(all_spans.size() * SPAN_INTS);
  for (size_t oi : order) {
    const Rec& r = recs[oi];
    s.tiles.insert(s.tiles.end(), {r.seg, r.q0, r.rows, s.n_spans(), r.nspan});
    for (int32_t k = 0; k < r.nspan; ++k) {
      const SpanOut& x = all_spans[r.span0 + k];
      s.spans.insert(s.spans.end(), {x.t0, x.t1, x.partial, 0});
    }
    s.tile_pairs += r.cost;
  }
}

// K/V-stationary schedule: for every K/V tile of every sub-sequence (up to the
// longest prefix of its two segments), the Q tiles of both segments that see it.
void build_kv_schedule(const Plan& p, const BlockSets& bs, Schedule& s, int32_t tile_q, int32_t tile_kv) {
  s.tile_q = tile_q;
  s.tile_kv = tile_kv;
  s.tiles.clear();
  s.spans.clear();
  s.tile_pairs = 0;
  struct Rec { int32_t seq, k0, keys, span0, nspan; int64_t cost; };
  struct Hit { int32_t seg, qt, partial; };
  std::vector<Rec> recs;
  std::vector<std::array<int32_t, 4>> all_spans;
  std::vector<int32_t> count, start;
  std::vector<Hit> hits;
  struct QSpan { int32_t seg, qt; SpanOut sp; };
  std::vector<QSpan> qspans;
  Scratch w;
  for (int32_t i = 0; i < p.n_seqs; ++i) {
    const int32_t segA = 2 * i, segB = 2 * i + 1;
    const int32_t kvmax = std::max(p.segs[segA * SEG_INTS + SEG_KVLEN], p.segs[segB * SEG_INTS + SEG_KVLEN]);
    const int32_t nkt = (kvmax + tile_kv - 1) / tile_kv;
    // pass 1: K/V spans of every Q tile of both segments (in segment, q tile order)
    qspans.clear();
    count.assign(nkt, 0);
    for (int32_t sg : {segA, segB}) {
      const int32_t q_len = p.segs[sg * SEG_INTS + SEG_QLEN];
      for (int32_t a0 = 0, qt = 0; a0 < q_len; a0 += tile_q, ++qt) {
        bs.tile(sg, a0, std::min(q_len, a0 + tile_q), w);
        tile_spans(w, tile_kv);
        // a Q tile that runs past the segment's end takes the element-wise
        // path, which also masks the rows past the end
        const bool short_tile = a0 + tile_q > q_len;
        for (SpanOut x : w.spans) {
          if (short_tile) x.partial = 1;
          qspans.push_back({sg, qt, x});
          for (int32_t t = x.t0; t < std::min(x.t1, nkt); ++t) ++count[t];
        }
      }
    }
    // pass 2: bucket the hits by K/V tile (CSR), keeping (segment, q tile) order
    start.assign(nkt + 1, 0);
    for (int32_t t = 0; t < nkt; ++t) start[t + 1] = start[t] + count[t];
    hits.resize(start[nkt]);
    std::fill(count.begin(), count.end(), 0);
    for (const QSpan& qs : qspans)
      for (int32_t t = qs.sp.t0; t < std::min(qs.sp.t1, nkt); ++t)
        hits[start[t] + count[t]++] = {qs.seg, qs.qt, qs.sp.partial};
    for (int32_t t = 0; t < nkt; ++t) {
      Rec r{i, t * tile_kv, std::min(tile_kv, kvmax - t * tile_kv), (int32_t)all_spans.size(), 0,
            (int64_t)(start[t + 1] - start[t])};
      for (int32_t h = start[t]; h < start[t + 1]; ++h) {
        const Hit& x = hits[h];
        if (r.nspan > 0) {
          auto& b = all_spans.back();
          if (b[0] == x.seg && b[2] == x.qt && b[3] == x.partial) { b[2] = x.qt + 1; continue; }
        }
        all_spans.push_back({x.seg, x.qt, x.qt + 1, x.partial});
        ++r.nspan;
      }
      recs.push_back(r);
    }
  }
  std::vector<size_t> order(recs.size());
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(),
                   [&](size_t x, size_t y) { return recs[x].cost > recs[y].cost; });
  s.tiles.reserve(recs.size() * KT_INTS);
  s.spans.reserve(all_spans.size() * SPAN_INTS);
  for (size_t oi : order) {
    const Rec& r = recs[oi];
    s.tiles.insert(s.tiles.end(), {r.seq, r.k0, r.keys, s.n_spans(), r.nspan});
    for (int32_t k = 0; k < r.nspan; ++k) {
      const auto& x = all_spans[r.span0 + k];
      s.spans.insert(s.spans.end(), x.begin(), x.end());
    }
    s.tile_pairs += r.cost;
  }
}

}  // namespace

void row_intervals(const Plan& p, int seg, int32_t a, int32_t iv[4]) {
  const int32_t* sg = &p.segs[(size_t)seg * SEG_INTS];
  position_intervals(p, sg[SEG_SEQ], sg[SEG_QPOS0] + a, iv);
}

void position_intervals(const Plan& p, int32_t seq, int32_t q, int32_t iv[4]) {
  iv[0] = 0; iv[1] = q + 1; iv[2] = 0; iv[3] = 0;
  if (p.mask_type == CVA_MASK_BLOCKWISE) {
    // DCP paper, sparse masks (Fig. 6(c)) and evaluation: blocks of `block`
    // tokens, `sink` leading blocks, a window of `window` blocks ending with the
    // query's own block, and the last block (the test sample) sees everything
    const int32_t L = p.cu[seq + 1] - p.cu[seq];
    const int32_t b = q / p.block;
    if (b != (L - 1) / p.block) {
      iv[1] = std::min((int64_t)p.sink * p.block, (int64_t)q + 1);
      iv[2] = std::max(0, (b - p.window + 1) * p.block);
      iv[3] = q + 1;
    }
  } else if (p.mask_type == CVA_MASK_LAMBDA) {
    iv[1] = std::min(p.sink, q + 1);
    iv[2] = std::max(0, q - p.window + 1);
    iv[3] = q + 1;
  } else if (p.mask_type == CVA_MASK_SHARED_PREFIX) {
    const int32_t nb = p.n_branches + 1;
    const int32_t* b = &p.branch_bounds[(size_t)seq * nb];
    if (q >= b[0]) {
      int32_t start = b[0];
      for (int32_t k = 1; k < nb; ++k) {
        if (q < b[k]) break;
        start = b[k];
      }
      iv[1] = b[0];
      iv[2] = start;
      iv[3] = q + 1;
    }
  }
}

FwdShape forward_shape(const Plan& p) {
  const int32_t G = p.hq / p.hkv;
  int32_t hpt = (G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1;
  FwdShape s;
  s.heads_per_tile = hpt;
  s.tile_q = kRowsPerWave * (kWavesPerFwdTile / hpt);
  s.tile_kv = kFwdTileKv;
  return s;
}

int32_t dq_tile_q(const Plan& p) {
  return kRowsPerWave * (kWavesPerDqTile / forward_shape(p).heads_per_tile);
}

cva_status build_schedules(Plan& p) {
  // per-row visible intervals and the useful pair count
  const int32_t nseg = (int32_t)(p.segs.size() / SEG_INTS);
  p.row_iv.assign((size_t)p.T_loc * 4, 0);
  // rows in chunks of 4096 (in parallel for large batches)
  std::vector<std::array<int32_t, 3>> chunks;  // (segment, first row, end row)
  for (int32_t sg = 0; sg < nseg; ++sg) {
    const int32_t q_len = p.segs[sg * SEG_INTS + SEG_QLEN];
    for (int32_t a0 = 0; a0 < q_len; a0 += 4096) chunks.push_back({sg, a0, std::min(q_len, a0 + 4096)});
  }
  std::vector<int64_t> chunk_pairs(chunks.size(), 0);
  parallel_for((int32_t)chunks.size(), p.T_loc, [&](int32_t c) {
    const int32_t sg = chunks[c][0];
    const int32_t row0 = p.segs[sg * SEG_INTS + SEG_QROW0];
    int64_t pairs = 0;
    for (int32_t a = chunks[c][1]; a < chunks[c][2]; ++a) {
      int32_t* iv = &p.row_iv[(size_t)(row0 + a) * 4];
      row_intervals(p, sg, a, iv);
      const RowSet rs = row_set(iv);
      for (int k = 0; k < rs.n; ++k) pairs += rs.v[k].second - rs.v[k].first;
    }
    chunk_pairs[c] = pairs;
  });
  p.visible_pairs = std::accumulate(chunk_pairs.begin(), chunk_pairs.end(), (int64_t)0);
  // visible pairs of every rank (RFC section 2: rank s holds chunks s and
  // 2R-1-s of every sub-sequence); rows are independent of the rank that holds them
  p.visible_pairs_per_rank.assign(p.cp_size, 0);
  if (p.cp_size == 1) p.visible_pairs_per_rank[0] = p.visible_pairs;
  for (int32_t i = 0; i < p.n_seqs && p.cp_size > 1; ++i) {
    const int32_t L = p.cu[i + 1] - p.cu[i];
    const int32_t c = L / (2 * p.cp_size);
    for (int32_t s = 0; s < p.cp_size; ++s) {
      for (int32_t j : {s, 2 * p.cp_size - 1 - s}) {
        for (int32_t q = j * c; q < (j + 1) * c; ++q) {
          int32_t iv[4];
          position_intervals(p, i, q, iv);
          const RowSet rs = row_set(iv);
          for (int k = 0; k < rs.n; ++k) p.visible_pairs_per_rank[s] += rs.v[k].second - rs.v[k].first;
        }
      }
    }
  }
  FwdShape fs = forward_shape(p);
  p.fwd_heads_per_tile = fs.heads_per_tile;
  BlockSets bs;
  bs.build(p);
  build_q_schedule(p, bs, p.fwd, fs.tile_q, fs.tile_kv);
  for (int32_t t = 0; t < p.fwd.n_tiles(); ++t) {
    if (p.fwd.tiles[(size_t)t * QT_INTS + QT_NSPAN] > kFwdMaxSpans) {
      set_error("mask gives a query tile more K/V spans than the forward kernel supports");
      return CVA_E_UNSUPPORTED;
    }
  }
  const int32_t dq_q = dq_tile_q(p);
  if (kDqTileKv == fs.tile_kv && dq_q == fs.tile_q)
    p.dq = p.fwd;  // same tile shape: the dQ kernel walks the forward schedule
  else
    build_q_schedule(p, bs, p.dq, dq_q, kDqTileKv);
  for (int32_t t = 0; t < p.dq.n_tiles(); ++t) {
    if (p.dq.tiles[(size_t)t * QT_INTS + QT_NSPAN] > kDqMaxSpans) {
      set_error("mask gives a query tile more K/V spans than the dQ kernel supports");
      return CVA_E_UNSUPPORTED;
    }
  }
  build_kv_schedule(p, bs, p.dkdv, kDkvTileQ, kDkvTileKv);
  for (int32_t t = 0; t < p.dkdv.n_tiles(); ++t) {
    if (p.dkdv.tiles[(size_t)t * KT_INTS + KT_NSPAN] > kDkvMaxSpans) {
      set_error("mask gives a K/V tile more query spans than the dK/dV kernel supports");
      return CVA_E_UNSUPPORTED;
    }
  }

  build_fwd_split(p);
  build_stream_deal(p, p.fwd, p.fwd_deal);
  build_stream_deal(p, p.fwds, p.fwds_deal);

  // rank-major rows outside every prefix are zero in dK/dV
  std::vector<char> covered((size_t)p.T, 0);
  for (int32_t x : p.kv_index) covered[x] = 1;
  // (in pieces of at most kZeroRowsPerBlock rows: one work-group each, so that
  // the zero fill spreads over the chip)
  p.zero_rows.clear();
  for (int64_t t = 0; t < p.T;) {
    if (covered[t]) { ++t; continue; }
    int64_t e = t;
    while (e < p.T && !covered[e]) ++e;
    for (int64_t a = t; a < e; a += kZeroRowsPerBlock) {
      p.zero_rows.push_back((int32_t)a);
      p.zero_rows.push_back((int32_t)std::min<int64_t>(e, a + kZeroRowsPerBlock));
    }
    t = e;
  }
  return CVA_OK;
}

void build_blob(Plan& p) {
  BlobLayout& L = p.layout;
  const std::vector<int32_t>* parts[] = {&p.segs, &p.kv_index, &p.row_iv, &p.fwd.tiles, &p.fwd.spans,
                                         &p.dq.tiles, &p.dq.spans, &p.dkdv.tiles, &p.dkdv.spans,
                                         &p.zero_rows, &p.fwds.tiles, &p.fwds.spans, &p.fwds_slot,
                                         &p.fwds_combine, &p.fwd_deal.start, &p.fwd_deal.items,
                                         &p.fwds_deal.start, &p.fwds_deal.items};
  int64_t* offs[] = {&L.segs, &L.kv_index, &L.row_iv, &L.fwd_tiles, &L.fwd_spans,
                     &L.dq_tiles, &L.dq_spans, &L.kv_tiles, &L.kv_spans, &L.zero_rows,
                     &L.fwds_tiles, &L.fwds_spans, &L.fwds_slot, &L.fwds_combine,
                     &L.fwd_deal_start, &L.fwd_deal_items, &L.fwds_deal_start, &L.fwds_deal_items};
  constexpr int kParts = (int)(sizeof(parts) / sizeof(parts[0]));
  int64_t total = 0;
  for (int k = 0; k < kParts; ++k) {
    *offs[k] = total;
    total += ((int64_t)parts[k]->size() + 63) / 64 * 64;  // every table 256-byte aligned
  }
  L.total = total;
  p.blob.assign((size_t)total, 0);
  for (int k = 0; k < kParts; ++k)
    if (!parts[k]->empty())
      std::memcpy(p.blob.data() + *offs[k], parts[k]->data(), parts[k]->size() * sizeof(int32_t));
}


// Forward schedule with split K/V ranges (DCP paper, background: the block-wise
// computation of one query block can be cut along the K/V dimension and the
// partial outputs merged through their log-sum-exp).  The forward's work items
// run one per CU (longest first); a Q tile whose K/V walk is much longer than
// the average work per CU bounds the whole launch, so such tiles are cut into
// pieces of at most `cap` K/V tiles (cap = that average, at least
// kSplitMinSteps), each piece an item of its own writing an fp32 partial result
// to its slot of the forward workspace.  When the average sets the cap, a tile
// is cut only if it walks more than 4/3 of it: the hardware's dispatch hands
// the next item to the first free CU, longest first, and such a list schedule
// already ends within 4/3 of the best one, so shorter tiles are not what bounds
// the launch (measured on MI355X: a packed 16k batch whose longest tile is 1.25x
// the average gains nothing from cutting; a sparse batch whose longest is 1.37x
// runs its forward 17 % faster cut).  A plan that cuts nothing needs no
// workspace.
void build_fwd_split(Plan& p) {
  p.fwds = Schedule{};
  p.fwds.tile_q = p.fwd.tile_q;
  p.fwds.tile_kv = p.fwd.tile_kv;
  p.fwds_slot.clear();
  p.fwds_combine.clear();
  p.n_split_slots = 0;
  const int32_t n = p.fwd.n_tiles();
  const int32_t groups = p.hq / p.fwd_heads_per_tile;
  std::vector<int64_t> steps(n, 0);
  int64_t total = 0;
  for (int32_t t = 0; t < n; ++t) {
    const int32_t* tr = &p.fwd.tiles[(size_t)t * QT_INTS];
    for (int32_t k = 0; k < tr[QT_NSPAN]; ++k) {
      const int32_t* sp = &p.fwd.spans[(size_t)(tr[QT_SPAN0] + k) * SPAN_INTS];
      steps[t] += sp[1] - sp[0];
    }
    total += steps[t] * groups;
  }
  int64_t cap = std::max<int64_t>(kSplitMinSteps, (total + kSplitCUs - 1) / kSplitCUs);
  int64_t cut_above = cap > kSplitMinSteps ? cap * 4 / 3 : cap;  // tiles walking more are cut
  // CVA_FWD_SPLIT_CAP in the environment replaces the cut length (K/V tiles per
  // piece, >= 1) and cuts every tile longer than it, e.g. to cut the long Q
  // tiles of a batch the default leaves whole
  if (const char* v = std::getenv("CVA_FWD_SPLIT_CAP")) {
    const long c = std::strtol(v, nullptr, 10);
    if (c >= 1) cap = cut_above = c;
  }
  p.fwd_split_cap = (int32_t)cap;
  struct Item { std::array<int32_t, QT_INTS> rec; std::vector<int32_t> spans; int32_t slot; int64_t cost; };
  std::vector<Item> items;
  for (int32_t t = 0; t < n; ++t) {
    const int32_t* tr = &p.fwd.tiles[(size_t)t * QT_INTS];
    std::vector<int32_t> sp(&p.fwd.spans[(size_t)tr[QT_SPAN0] * SPAN_INTS],
                            &p.fwd.spans[(size_t)(tr[QT_SPAN0] + tr[QT_NSPAN]) * SPAN_INTS]);
    const int64_t pieces =
        steps[t] > cut_above ? std::min<int64_t>(kSplitMaxPieces, (steps[t] + cap - 1) / cap) : 1;
    if (pieces <= 1) {
      items.push_back({{tr[0], tr[1], tr[2], 0, tr[QT_NSPAN]}, sp, -1, steps[t]});
      continue;
    }
    p.fwds_combine.insert(p.fwds_combine.end(),
                          {tr[QT_SEG], tr[QT_Q0], tr[QT_ROWS], p.n_split_slots, (int32_t)pieces});
    // cut the K/V tiles of the span list into `pieces` consecutive runs of
    // near-equal length (a span may be cut in the middle)
    int64_t done = 0;
    size_t k = 0;
    int32_t pos = sp.empty() ? 0 : sp[0];  // next K/V tile of span k
    for (int64_t i = 0; i < pieces; ++i) {
      const int64_t want = steps[t] * (i + 1) / pieces - done;
      Item it{{tr[0], tr[1], tr[2], 0, 0}, {}, p.n_split_slots + (int32_t)i, want};
      int64_t got = 0;
      while (got < want) {
        const int32_t end = sp[k * SPAN_INTS + 1];
        const int32_t take = (int32_t)std::min<int64_t>(end - pos, want - got);
        it.spans.insert(it.spans.end(), {pos, pos + take, sp[k * SPAN_INTS + 2], 0});
        ++it.rec[QT_NSPAN];
        pos += take;
        got += take;
        if (pos == end && k + 1 < sp.size() / SPAN_INTS) {
          ++k;
          pos = sp[k * SPAN_INTS];
        }
      }
      done += got;
      items.push_back(std::move(it));
    }
    p.n_split_slots += (int32_t)pieces;
  }
  std::stable_sort(items.begin(), items.end(), [](const Item& a, const Item& b) { return a.cost > b.cost; });
  for (Item& it : items) {
    it.rec[QT_SPAN0] = p.fwds.n_spans();
    p.fwds.tiles.insert(p.fwds.tiles.end(), it.rec.begin(), it.rec.end());
    p.fwds.spans.insert(p.fwds.spans.end(), it.spans.begin(), it.spans.end());
    p.fwds_slot.push_back(it.slot);
    p.fwds.tile_pairs += it.cost;
  }
}

void build_stream_deal(const Plan& p, const Schedule& s, StreamDeal& d) {
  d = StreamDeal{};
  const int32_t n = s.n_tiles();
  if (n == 0 || p.dtype == CVA_FP32) return;
  const int32_t groups = p.hq / p.fwd_heads_per_tile;
  int32_t wgs = std::min<int32_t>(n, std::max<int32_t>(1, kSplitCUs / groups));
  // CVA_FWD_STREAM_WGS in the environment caps the work-groups per head group
  // (>= 1), e.g. to give every work-group of a small batch several items
  if (const char* v = std::getenv("CVA_FWD_STREAM_WGS")) {
    const long c = std::strtol(v, nullptr, 10);
    if (c >= 1) wgs = std::min<int32_t>(wgs, (int32_t)c);
  }
  if ((n + wgs - 1) / wgs > kFwdStreamMaxItems) return;  // more rounds than the LDS table holds
  // Round by round (each work-group one item per round, so that the work-groups
  // of an XCD start their items together and walk the same K/V tiles at about
  // the same time), the round's items in schedule order (longest first) to the
  // work-groups in order of their load so far (least loaded first).
  std::vector<std::vector<int32_t>> lists((size_t)wgs);
  std::vector<int64_t> load((size_t)wgs, 0);
  std::vector<int32_t> order((size_t)wgs);
  for (int32_t r0 = 0; r0 < n; r0 += wgs) {
    std::iota(order.begin(), order.end(), 0);
    std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) { return load[(size_t)a] < load[(size_t)b]; });
    for (int32_t k = 0; k < wgs && r0 + k < n; ++k) {
      const int32_t t = r0 + k;
      const int32_t* tr = &s.tiles[(size_t)t * QT_INTS];
      int64_t steps = kStreamItemSteps;
      for (int32_t j = 0; j < tr[QT_NSPAN]; ++j) {
        const int32_t* sp = &s.spans[(size_t)(tr[QT_SPAN0] + j) * SPAN_INTS];
        steps += sp[1] - sp[0];
      }
      const int32_t w = order[(size_t)k];
      lists[(size_t)w].push_back(t);
      load[(size_t)w] += steps;
    }
  }
  d.wgs = wgs;
  d.start.assign(1, 0);
  for (const auto& li : lists) {
    d.items.insert(d.items.end(), li.begin(), li.end());
    d.start.push_back((int32_t)d.items.size());
  }
}

}  // namespace cva

namespace cva {

// Forward items of a placed plan: for every Q tile of every segment (Q block)
// and every computation block of that segment, the K/V tiles of the block's
// key range that the tile's rows see, as one item with a partial slot of its
// own; one merge record per Q tile lists its consecutive slots (possibly none:
// the merge then gives its rows O = 0 and LSE = -inf, no visible key).
cva_status build_placed_schedule(Plan& p, const std::vector<PlacedBlock>& blocks) {
  const FwdShape fs = forward_shape(p);
  p.fwd_heads_per_tile = fs.heads_per_tile;
  p.fwd = p.dq = p.dkdv = Schedule{};
  p.fwd.tile_q = p.dq.tile_q = fs.tile_q;
  p.fwd.tile_kv = p.dq.tile_kv = fs.tile_kv;
  p.dkdv.tile_q = kDkvTileQ;
  p.dkdv.tile_kv = kDkvTileKv;
  p.fwds = Schedule{};
  p.fwds.tile_q = fs.tile_q;
  p.fwds.tile_kv = fs.tile_kv;
  p.fwds_slot.clear();
  p.fwds_combine.clear();
  p.zero_rows.clear();
  p.n_split_slots = 0;
  p.fwd_split_cap = 0;
  struct Item { std::array<int32_t, QT_INTS> rec; std::vector<SpanOut> spans; int32_t slot; int64_t cost; };
  std::vector<Item> items;
  Scratch w;
  IvList U0, F0;
  const int32_t nseg = (int32_t)(p.segs.size() / SEG_INTS);
  size_t b0 = 0;
  for (int32_t sg = 0; sg < nseg; ++sg) {
    size_t b1 = b0;
    while (b1 < blocks.size() && blocks[b1].seg == sg) ++b1;
    const int32_t q_len = p.segs[(size_t)sg * SEG_INTS + SEG_QLEN];
    for (int32_t a0 = 0; a0 < q_len; a0 += fs.tile_q) {
      const int32_t a1 = std::min(q_len, a0 + fs.tile_q);
      tile_sets(p, sg, a0, a1, w);
      U0 = w.U;
      F0 = w.F;
      const int32_t slot0 = p.n_split_slots;
      for (size_t b = b0; b < b1; ++b) {
        const int32_t k0 = blocks[b].k0, k1 = blocks[b].k1;
        auto clip = [&](const IvList& in, IvList& out) {
          out.clear();
          for (const Iv& x : in) {
            const int32_t lo = std::max(x.first, k0), hi = std::min(x.second, k1);
            if (hi > lo) out.push_back({lo, hi});
          }
        };
        clip(U0, w.U);
        clip(F0, w.F);
        tile_spans(w, fs.tile_kv);
        if (w.spans.empty()) continue;  // no row of this tile sees a key of the block
        if ((int32_t)w.spans.size() > kFwdMaxSpans) {
          set_error("a computation block gives a query tile more K/V spans than the forward kernel supports");
          return CVA_E_UNSUPPORTED;
        }
        Item it{{sg, a0, a1 - a0, 0, (int32_t)w.spans.size()}, w.spans, p.n_split_slots++, 0};
        for (const SpanOut& x : w.spans) it.cost += x.t1 - x.t0;
        items.push_back(std::move(it));
      }
      p.fwds_combine.insert(p.fwds_combine.end(), {sg, a0, a1 - a0, slot0, p.n_split_slots - slot0});
    }
    b0 = b1;
  }
  std::stable_sort(items.begin(), items.end(), [](const Item& a, const Item& b) { return a.cost > b.cost; });
  for (Item& it : items) {
    it.rec[QT_SPAN0] = p.fwds.n_spans();
    p.fwds.tiles.insert(p.fwds.tiles.end(), it.rec.begin(), it.rec.end());
    for (const SpanOut& x : it.spans) p.fwds.spans.insert(p.fwds.spans.end(), {x.t0, x.t1, x.partial, 0});
    p.fwds_slot.push_back(it.slot);
    p.fwds.tile_pairs += it.cost;
  }
  p.fwd_deal = StreamDeal{};
  build_stream_deal(p, p.fwds, p.fwds_deal);
  return CVA_OK;
}

}  // namespace cva
