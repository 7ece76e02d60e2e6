// Block-ALS path (placeholder until the MFMA kernels land).
#include "externd_internal.hpp"

namespace externd {

size_t block_workspace_bytes(int, int, int) { return 256; }

hipError_t block_run(const BlockLaunch&, hipStream_t, double*) { return hipErrorNotSupported; }

}  // namespace externd
