// chunk_bwd_mfma.hip -- dispatch of the bf16 matrix-core backward (chunk_bwd_mfma_impl.h) over the
// head dims it serves, each instantiated in its own translation unit (chunk_bwd_mfma_d<D>.hip).
#include "la_device.h"
#include "la_internal.h"

namespace la {

hipError_t launch_bwd_mfma_d32(const BwdArgs& a);
hipError_t launch_bwd_mfma_d64(const BwdArgs& a);
hipError_t launch_bwd_mfma_d128(const BwdArgs& a);

bool chunk_bwd_mfma_supported(const BwdArgs& a) {
    return a.bf16 && a.dk == a.dv && (a.dk == 32 || a.dk == 64 || a.dk == 128) && a.chunk == 64 && a.L > 0 &&
           a.B * a.H > 0 && (a.mode == DECAY_NONE || a.mode == DECAY_HEAD || a.mode == DECAY_GATE);
}

hipError_t launch_chunk_bwd_mfma(const BwdArgs& a) {
    if (a.dk == 128) return launch_bwd_mfma_d128(a);
    if (a.dk == 64) return launch_bwd_mfma_d64(a);
    return launch_bwd_mfma_d32(a);
}

}  // namespace la
