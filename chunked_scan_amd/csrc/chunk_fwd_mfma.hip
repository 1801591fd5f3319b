// chunk_fwd_mfma.hip -- placeholder dispatch while the bf16 MFMA kernels are written.
#include "la_device.h"
#include "la_internal.h"

namespace la {
hipError_t launch_chunk_fwd_mfma(const FwdArgs& a) { return launch_chunk_fwd_generic(a); }
hipError_t launch_state_correct(const CorrectArgs& a) { return launch_state_correct_generic(a); }
}  // namespace la
