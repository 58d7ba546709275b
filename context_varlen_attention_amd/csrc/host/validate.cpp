// Request validation, run before any metadata or device work.
//
// The checks follow the MindSpeed RFC (issue 232): usage limits of section 2
// (positive sub-sequences divisible by 2*CP, Hq a multiple of Hkv, Dq == Dk,
// Dk >= Dv), the parameter ranges of get_thd_load_balanced_cp_metadata in
// section 3.5.2.1 (cu_seqlens non-empty and strictly increasing, cp_size >= 1,
// rank in [0, cp_size)) and the "fail early, before communication or operator
// calls" rule of section 3.4.  Each failure class has its own status code.
#include <climits>
#include <sstream>

#include "plan.hpp"

namespace cva {

namespace {
thread_local std::string g_err;
}

void set_error(const std::string& msg) { g_err = msg; }
const char* last_error() { return g_err.c_str(); }

static cva_status fail(cva_status s, const std::string& msg) {
  set_error(msg);
  return s;
}

bool head_dims_supported(int32_t /*dtype*/, int32_t d_qk, int32_t d_v) {
  return (d_qk == 64 && d_v == 64) || (d_qk == 128 && d_v == 128) || (d_qk == 192 && d_v == 128);
}

cva_status validate_mask(const cva_mask_desc* mask, const int32_t* cu, int32_t n_seqs) {
  if (mask != nullptr) {
    switch (mask->type) {
      case CVA_MASK_CAUSAL:
        break;
      case CVA_MASK_LAMBDA:
        if (mask->sink < 0 || mask->window < 1)
          return fail(CVA_E_MASK, "lambda mask needs sink >= 0 and window >= 1");
        break;
      case CVA_MASK_SHARED_PREFIX: {
        if (mask->n_branches < 1 || mask->branch_bounds == nullptr)
          return fail(CVA_E_MASK, "shared-prefix mask needs n_branches >= 1 and branch_bounds");
        const int32_t nb = mask->n_branches + 1;
        for (int32_t i = 0; i < n_seqs; ++i) {
          const int32_t* b = mask->branch_bounds + (int64_t)i * nb;
          int32_t L = cu[i + 1] - cu[i];
          if (b[0] < 0) return fail(CVA_E_MASK, "shared-prefix bounds must be >= 0");
          for (int32_t k = 1; k < nb; ++k)
            if (b[k] < b[k - 1]) return fail(CVA_E_MASK, "shared-prefix bounds must be non-decreasing");
          if (b[nb - 1] != L)
            return fail(CVA_E_MASK, "last shared-prefix bound must equal the sub-sequence length");
        }
        break;
      }
      case CVA_MASK_BLOCKWISE:
        if (mask->block < 1 || mask->sink < 0 || mask->window < 1)
          return fail(CVA_E_MASK, "blockwise mask needs block >= 1, sink >= 0 and window >= 1 (blocks)");
        break;
      default:
        return fail(CVA_E_MASK, "unknown mask type");
    }
  }
  return CVA_OK;
}

cva_status validate_request(const int32_t* cu, int32_t n_seqs, int32_t cp_size, int32_t rank,
                            const cva_mask_desc* mask, int32_t hq, int32_t hkv, int32_t d_qk,
                            int32_t d_v, int32_t dtype) {
  if (cu == nullptr) return fail(CVA_E_ARG, "cu_seqlens is NULL");
  if (n_seqs < 1) return fail(CVA_E_CU_SEQLENS, "cu_seqlens must hold at least one sub-sequence");
  if (cp_size < 1) return fail(CVA_E_RANK, "cp_size must be >= 1");
  if (rank < 0 || rank >= cp_size) return fail(CVA_E_RANK, "rank must be in [0, cp_size)");
  if (cu[0] != 0) return fail(CVA_E_CU_SEQLENS, "cu_seqlens must start at 0");
  for (int32_t i = 0; i < n_seqs; ++i) {
    int64_t L = (int64_t)cu[i + 1] - cu[i];
    if (L <= 0) {
      std::ostringstream os;
      os << "cu_seqlens must be strictly increasing (sub-sequence " << i << " has length " << L << ")";
      return fail(CVA_E_CU_SEQLENS, os.str());
    }
    if (L % (2 * (int64_t)cp_size) != 0) {
      std::ostringstream os;
      os << "sub-sequence " << i << " of length " << L << " is not divisible by 2*cp_size = "
         << 2 * cp_size;
      return fail(CVA_E_ALIGN, os.str());
    }
  }
  // kv_index holds T*(2R+1)/(2R) int32 entries; keep every count inside int32.
  int64_t T = cu[n_seqs];
  if (T > INT32_MAX / 2) return fail(CVA_E_UNSUPPORTED, "total tokens too large for int32 indexing");
  if (hq < 1 || hkv < 1) return fail(CVA_E_HEADS, "head counts must be >= 1");
  if (hq % hkv != 0) return fail(CVA_E_HEADS, "query heads must be a multiple of K/V heads");
  if (dtype != CVA_BF16 && dtype != CVA_FP16 && dtype != CVA_FP32)
    return fail(CVA_E_DTYPE, "dtype must be CVA_BF16, CVA_FP16 or CVA_FP32");
  if (d_qk < 1 || d_v < 1 || d_qk < d_v)
    return fail(CVA_E_HEADDIM, "head dims must satisfy Dqk >= Dv >= 1");
  if (!head_dims_supported(dtype, d_qk, d_v)) {
    std::ostringstream os;
    os << "no kernel for (Dqk, Dv) = (" << d_qk << ", " << d_v
       << "); supported: (64,64), (128,128), (192,128)";
    return fail(CVA_E_HEADDIM, os.str());
  }
  return validate_mask(mask, cu, n_seqs);
}

}  // namespace cva
