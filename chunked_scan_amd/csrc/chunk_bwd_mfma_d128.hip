// chunk_bwd_mfma_d128.hip -- the bf16 matrix-core backward (chunk_bwd_mfma_impl.h) for dk = dv = 128.
#include "chunk_bwd_mfma_impl.h"

namespace la {

hipError_t launch_bwd_mfma_d128(const BwdArgs& a) { return launch_d<128>(a); }

}  // namespace la
