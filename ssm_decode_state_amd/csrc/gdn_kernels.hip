// gdn_kernels.hip -- Gated DeltaNet ReplaySSM kernels for gfx950 (not yet implemented).
#include "ssm_device.hpp"
#include "ssm_kernels.hpp"

namespace ssm {

hipError_t gdn_launch_replay(const GdnArgs&, int, int, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t gdn_launch_flush(const GdnArgs&, int, int, int, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t gdn_launch_conv(const GdnConvArgs&, int, int, int, hipStream_t) { return hipErrorNotSupported; }

}  // namespace ssm
