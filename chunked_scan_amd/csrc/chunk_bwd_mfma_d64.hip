// chunk_bwd_mfma_d64.hip -- the bf16 matrix-core backward (chunk_bwd_mfma_impl.h) for dk = dv = 64.
#include "chunk_bwd_mfma_impl.h"

namespace la {

hipError_t launch_bwd_mfma_d64(const BwdArgs& a) { return launch_d<64>(a); }

}  // namespace la
