// Metadata builder: from (cu_seqlens, cp_size R, rank r) to the token counts,
// cumulative Q/KV lengths and the rank-major causal-prefix index.
//
// MindSpeed RFC (issue 232): section 2 fixes the split (2R chunks per EOD
// sub-sequence, rank r holds chunks r and 2R-1-r) and the balance criterion
// sum(q_len*kv_len); section 3.1 lists what the builder returns (local and
// global token counts, actual_seq_qlen / actual_seq_kvlen for the fused call,
// and the index that selects each chunk's causal K/V prefix from the
// rank-major all-gathered K/V).
//
// Layout readings (the page leaves them open): a rank's local rows run
// sub-sequence by sub-sequence, chunk r first, then chunk 2R-1-r; cumulative
// lengths carry a leading 0; a chunk-j segment's prefix is positions
// 0..(j+1)c-1 of its sub-sequence, in order.
//
// The index is computed in closed form: position p of sub-sequence i lies in
// chunk j = p / c at offset o = p % c; chunk j belongs to rank j (first local
// chunk, local offset o) when j < R, else to rank 2R-1-j (second local chunk,
// local offset c + o); its rank-major row is rank * T_loc + cu[i]/R + offset.
#include <sstream>

#include "plan.hpp"

namespace cva {

cva_status build_metadata(Plan& p) {
  const int32_t n = p.n_seqs, R = p.cp_size, r = p.rank;
  p.T = p.cu[n];
  p.T_loc = p.T / R;
  const int64_t T_loc = p.T_loc;

  p.local_cu.assign(n + 1, 0);
  for (int32_t i = 0; i <= n; ++i) p.local_cu[i] = p.cu[i] / R;

  p.aq.assign(1, 0);
  p.akv.assign(1, 0);
  p.seg_q_pos0.clear();
  p.segs.clear();
  p.kv_index.clear();
  p.kv_index.reserve((size_t)(p.T + p.T / (2 * R)));

  for (int32_t i = 0; i < n; ++i) {
    const int32_t L = p.cu[i + 1] - p.cu[i];
    const int32_t c = L / (2 * R);
    const int32_t lcu = p.local_cu[i];
    const int32_t chunks[2] = {r, 2 * R - 1 - r};
    for (int32_t e = 0; e < 2; ++e) {
      const int32_t j = chunks[e];
      const int32_t q_len = c, kv_len = (j + 1) * c;
      int32_t seg[SEG_INTS];
      seg[SEG_SEQ] = i;
      seg[SEG_CHUNK] = j;
      seg[SEG_QLEN] = q_len;
      seg[SEG_KVLEN] = kv_len;
      seg[SEG_QROW0] = p.aq.back();
      seg[SEG_KVOFF] = p.akv.back();
      seg[SEG_QPOS0] = j * c;
      seg[SEG_SEQLEN] = L;
      p.segs.insert(p.segs.end(), seg, seg + SEG_INTS);
      p.aq.push_back(p.aq.back() + q_len);
      p.akv.push_back(p.akv.back() + kv_len);
      p.seg_q_pos0.push_back(j * c);
      // prefix positions 0..kv_len-1, one chunk (a contiguous rank-major run) at a time
      for (int32_t jj = 0; jj <= j; ++jj) {
        const int32_t owner = jj < R ? jj : 2 * R - 1 - jj;
        const int32_t off = jj < R ? 0 : c;
        const int64_t base = (int64_t)owner * T_loc + lcu + off;
        for (int32_t o = 0; o < c; ++o) p.kv_index.push_back((int32_t)(base + o));
      }
    }
  }

  // per-rank workload sum(q_len * kv_len), each rank's segments taken on their own
  p.workload.assign(R, 0);
  for (int32_t s = 0; s < R; ++s) {
    int64_t w = 0;
    for (int32_t i = 0; i < n; ++i) {
      const int64_t c = (p.cu[i + 1] - p.cu[i]) / (2 * R);
      w += c * ((int64_t)(s + 1) * c) + c * ((int64_t)(2 * R - s) * c);
    }
    p.workload[s] = w;
  }
  for (int32_t s = 1; s < R; ++s) {
    if (p.workload[s] != p.workload[0]) {
      std::ostringstream os;
      os << "per-rank workload differs: rank 0 has " << p.workload[0] << ", rank " << s << " has "
         << p.workload[s];
      set_error(os.str());
      return CVA_E_WORKLOAD;
    }
  }
  return CVA_OK;
}

}  // namespace cva
