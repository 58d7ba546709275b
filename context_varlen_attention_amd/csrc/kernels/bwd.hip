// Backward attention kernels for gfx950 (placeholder until the MFMA backward lands).
#include "common.hpp"
#include "launch.hpp"

namespace cva {

hipError_t launch_bwd(int, int, int, const BwdParams&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace cva
