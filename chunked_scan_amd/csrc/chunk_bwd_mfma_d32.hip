// chunk_bwd_mfma_d32.hip -- the bf16 matrix-core backward (chunk_bwd_mfma_impl.h) for dk = dv = 32.
#include "chunk_bwd_mfma_impl.h"

namespace la {

hipError_t launch_bwd_mfma_d32(const BwdArgs& a) { return launch_d<32>(a); }

}  // namespace la
