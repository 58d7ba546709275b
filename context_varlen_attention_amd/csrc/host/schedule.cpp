// Block-mask tile scheduler.
//
// DCP paper (block-wise attention and its computation blocks): a computation
// block pairs a Q block with a K/V block and is only created where the mask
// between them is not all zero, so masked work is discarded before it is
// launched.  This file does that on kernel tiles.
//
// Every query row's visible keys form at most two intervals of in-sequence
// positions (row_intervals): causal [0, q]; lambda [0, min(sink, q+1)) and
// [q-window+1, q] (DCP Fig. 6(b)); shared prefix [0, q] inside the question,
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
#include <numeric>

#include "plan.hpp"

namespace cva {

namespace {

using Iv = std::pair<int32_t, int32_t>;  // [first, end)
using IvList = std::vector<Iv>;

IvList normalize(IvList v) {
  v.erase(std::remove_if(v.begin(), v.end(), [](const Iv& x) { return x.second <= x.first; }),
          v.end());
  std::sort(v.begin(), v.end());
  IvList out;
  for (const Iv& x : v) {
    if (!out.empty() && x.first <= out.back().second)
      out.back().second = std::max(out.back().second, x.second);
    else
      out.push_back(x);
  }
  return out;
}

IvList intersect(const IvList& a, const IvList& b) {
  IvList out;
  size_t i = 0, j = 0;
  while (i < a.size() && j < b.size()) {
    int32_t lo = std::max(a[i].first, b[j].first);
    int32_t hi = std::min(a[i].second, b[j].second);
    if (hi > lo) out.push_back({lo, hi});
    if (a[i].second < b[j].second) ++i; else ++j;
  }
  return out;
}

IvList row_set(const Plan& p, int seg, int32_t a) {
  int32_t iv[4];
  row_intervals(p, seg, a, iv);
  return normalize({{iv[0], iv[1]}, {iv[2], iv[3]}});
}

struct SpanOut {
  int32_t t0, t1, partial;
};

// Spans of tiles of width `bn` given the union U and intersection F of the rows' visible sets.
std::vector<SpanOut> tile_spans(const IvList& U, const IvList& F, int32_t bn) {
  std::vector<Iv> ne;  // non-empty tile ranges
  for (const Iv& u : U) {
    int32_t t0 = u.first / bn, t1 = (u.second + bn - 1) / bn;
    if (!ne.empty() && t0 <= ne.back().second)
      ne.back().second = std::max(ne.back().second, t1);
    else
      ne.push_back({t0, t1});
  }
  std::vector<Iv> full;
  for (const Iv& f : F) {
    int32_t t0 = (f.first + bn - 1) / bn, t1 = f.second / bn;
    if (t1 > t0) full.push_back({t0, t1});
  }
  std::vector<SpanOut> out;
  size_t k = 0;
  for (const Iv& r : ne) {
    int32_t cur = r.first;
    while (k < full.size() && full[k].second <= cur) ++k;
    while (k < full.size() && full[k].first < r.second) {
      int32_t f0 = std::max(full[k].first, cur), f1 = std::min(full[k].second, r.second);
      if (f0 > cur) out.push_back({cur, f0, 1});
      if (f1 > f0) out.push_back({f0, f1, 0});
      cur = std::max(cur, f1);
      if (full[k].second <= r.second) ++k; else break;
    }
    if (cur < r.second) out.push_back({cur, r.second, 1});
  }
  return out;
}

// Union and intersection of the visible sets of rows [a0, a1) of a segment.
void tile_sets(const Plan& p, int seg, int32_t a0, int32_t a1, IvList& U, IvList& F) {
  IvList all;
  F.clear();
  for (int32_t a = a0; a < a1; ++a) {
    IvList s = row_set(p, seg, a);
    all.insert(all.end(), s.begin(), s.end());
    F = (a == a0) ? s : intersect(F, s);
  }
  U = normalize(all);
}

void build_q_schedule(const Plan& p, Schedule& s, int32_t tile_q, int32_t tile_kv) {
  s.tile_q = tile_q;
  s.tile_kv = tile_kv;
  s.tiles.clear();
  s.spans.clear();
  s.tile_pairs = 0;
  struct Rec { int32_t seg, q0, rows; std::vector<SpanOut> sp; int64_t cost; };
  std::vector<Rec> recs;
  const int32_t nseg = (int32_t)(p.segs.size() / SEG_INTS);
  for (int32_t sg = 0; sg < nseg; ++sg) {
    const int32_t q_len = p.segs[sg * SEG_INTS + SEG_QLEN];
    for (int32_t a0 = 0; a0 < q_len; a0 += tile_q) {
      const int32_t a1 = std::min(q_len, a0 + tile_q);
      IvList U, F;
      tile_sets(p, sg, a0, a1, U, F);
      Rec r{sg, a0, a1 - a0, tile_spans(U, F, tile_kv), 0};
      for (const SpanOut& x : r.sp) r.cost += x.t1 - x.t0;
      recs.push_back(std::move(r));
    }
  }
  std::vector<size_t> order(recs.size());
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(),
                   [&](size_t x, size_t y) { return recs[x].cost > recs[y].cost; });
  for (size_t oi : order) {
    const Rec& r = recs[oi];
    s.tiles.insert(s.tiles.end(),
                   {r.seg, r.q0, r.rows, s.n_spans(), (int32_t)r.sp.size()});
    for (const SpanOut& x : r.sp) s.spans.insert(s.spans.end(), {x.t0, x.t1, x.partial, 0});
    s.tile_pairs += r.cost;
  }
}

// K/V-stationary schedule: for every K/V tile of every sub-sequence (up to the
// longest prefix of its two segments), the Q tiles of both segments that see it.
void build_kv_schedule(const Plan& p, Schedule& s, int32_t tile_q, int32_t tile_kv) {
  s.tile_q = tile_q;
  s.tile_kv = tile_kv;
  s.tiles.clear();
  s.spans.clear();
  s.tile_pairs = 0;
  struct Rec { int32_t seq, k0, keys; std::vector<std::array<int32_t, 4>> sp; int64_t cost; };
  std::vector<Rec> recs;
  for (int32_t i = 0; i < p.n_seqs; ++i) {
    const int32_t segA = 2 * i, segB = 2 * i + 1;
    const int32_t kvmax = std::max(p.segs[segA * SEG_INTS + SEG_KVLEN], p.segs[segB * SEG_INTS + SEG_KVLEN]);
    const int32_t nkt = (kvmax + tile_kv - 1) / tile_kv;
    // per K/V tile: list of (segment, q tile, partial)
    std::vector<std::vector<std::array<int32_t, 3>>> hits(nkt);
    for (int32_t sg : {segA, segB}) {
      const int32_t q_len = p.segs[sg * SEG_INTS + SEG_QLEN];
      for (int32_t a0 = 0, qt = 0; a0 < q_len; a0 += tile_q, ++qt) {
        IvList U, F;
        tile_sets(p, sg, a0, std::min(q_len, a0 + tile_q), U, F);
        for (const SpanOut& x : tile_spans(U, F, tile_kv))
          for (int32_t t = x.t0; t < x.t1 && t < nkt; ++t) hits[t].push_back({sg, qt, x.partial});
      }
    }
    for (int32_t t = 0; t < nkt; ++t) {
      Rec r{i, t * tile_kv, std::min(tile_kv, kvmax - t * tile_kv), {}, (int64_t)hits[t].size()};
      for (const auto& h : hits[t]) {
        if (!r.sp.empty() && r.sp.back()[0] == h[0] && r.sp.back()[2] == h[1] && r.sp.back()[3] == h[2])
          r.sp.back()[2] = h[1] + 1;
        else
          r.sp.push_back({h[0], h[1], h[1] + 1, h[2]});
      }
      recs.push_back(std::move(r));
    }
  }
  std::vector<size_t> order(recs.size());
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(),
                   [&](size_t x, size_t y) { return recs[x].cost > recs[y].cost; });
  for (size_t oi : order) {
    const Rec& r = recs[oi];
    s.tiles.insert(s.tiles.end(), {r.seq, r.k0, r.keys, s.n_spans(), (int32_t)r.sp.size()});
    for (const auto& x : r.sp) s.spans.insert(s.spans.end(), x.begin(), x.end());
    s.tile_pairs += r.cost;
  }
}

}  // namespace

void row_intervals(const Plan& p, int seg, int32_t a, int32_t iv[4]) {
  const int32_t* sg = &p.segs[(size_t)seg * SEG_INTS];
  const int32_t q = sg[SEG_QPOS0] + a;
  iv[0] = 0; iv[1] = q + 1; iv[2] = 0; iv[3] = 0;
  if (p.mask_type == CVA_MASK_LAMBDA) {
    iv[1] = std::min(p.sink, q + 1);
    iv[2] = std::max(0, q - p.window + 1);
    iv[3] = q + 1;
  } else if (p.mask_type == CVA_MASK_SHARED_PREFIX) {
    const int32_t nb = p.n_branches + 1;
    const int32_t* b = &p.branch_bounds[(size_t)sg[SEG_SEQ] * nb];
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

cva_status build_schedules(Plan& p) {
  // per-row visible intervals and the useful pair count
  const int32_t nseg = (int32_t)(p.segs.size() / SEG_INTS);
  p.row_iv.assign((size_t)p.T_loc * 4, 0);
  p.visible_pairs = 0;
  for (int32_t sg = 0; sg < nseg; ++sg) {
    const int32_t q_len = p.segs[sg * SEG_INTS + SEG_QLEN];
    const int32_t row0 = p.segs[sg * SEG_INTS + SEG_QROW0];
    for (int32_t a = 0; a < q_len; ++a) {
      int32_t* iv = &p.row_iv[(size_t)(row0 + a) * 4];
      row_intervals(p, sg, a, iv);
      for (const Iv& x : normalize({{iv[0], iv[1]}, {iv[2], iv[3]}})) p.visible_pairs += x.second - x.first;
    }
  }
  FwdShape fs = forward_shape(p);
  p.fwd_heads_per_tile = fs.heads_per_tile;
  build_q_schedule(p, p.fwd, fs.tile_q, fs.tile_kv);
  build_q_schedule(p, p.dq, fs.tile_q, kDqTileKv);
  build_kv_schedule(p, p.dkdv, kDkvTileQ, kDkvTileKv);

  // rank-major rows outside every prefix are zero in dK/dV
  std::vector<char> covered((size_t)p.T, 0);
  for (int32_t x : p.kv_index) covered[x] = 1;
  p.zero_rows.clear();
  for (int64_t t = 0; t < p.T;) {
    if (covered[t]) { ++t; continue; }
    int64_t e = t;
    while (e < p.T && !covered[e]) ++e;
    p.zero_rows.push_back((int32_t)t);
    p.zero_rows.push_back((int32_t)e);
    t = e;
  }
  return CVA_OK;
}

void build_blob(Plan& p) {
  BlobLayout& L = p.layout;
  std::vector<int32_t>& b = p.blob;
  b.clear();
  auto put = [&](const std::vector<int32_t>& v) {
    int64_t off = (int64_t)b.size();
    b.insert(b.end(), v.begin(), v.end());
    while (b.size() % 64) b.push_back(0);  // keep every table 256-byte aligned
    return off;
  };
  L.segs = put(p.segs);
  L.kv_index = put(p.kv_index);
  L.row_iv = put(p.row_iv);
  L.fwd_tiles = put(p.fwd.tiles);
  L.fwd_spans = put(p.fwd.spans);
  L.dq_tiles = put(p.dq.tiles);
  L.dq_spans = put(p.dq.spans);
  L.kv_tiles = put(p.dkdv.tiles);
  L.kv_spans = put(p.dkdv.spans);
  L.zero_rows = put(p.zero_rows);
  L.total = (int64_t)b.size();
}

}  // namespace cva
