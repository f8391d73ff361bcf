// Ragged and paged prefill attention (MFMA). Not built yet: both launchers report "not supported".
#include "common.h"
#include "kernels.h"

namespace pkv {

hipError_t launch_ragged_prefill(const PrefillArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_paged_prefill(const PrefillArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace pkv
