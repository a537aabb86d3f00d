// launch_stub.cpp -- the kernel launchers of launch.hpp for a host-only build
// of the C ABI (kvc_api.cpp) under AddressSanitizer and UBSan.  Test
// infrastructure: no device code is built, so every launcher reports that
// no device can run it, and a call that gets past its host-side checks
// returns KVC_ELAUNCH.  The CPU tests only make calls that return before any
// launch.
#include "../../fp8_fp4_quantized_amd/csrc/launch.hpp"

namespace kvc {

hipError_t launch_store_rows(const StoreParams&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_dequant_gather(const GatherParams&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_compress(const CompressParams&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_dcp_filter(const DcpFilterParams&, hipStream_t) { return hipErrorNoDevice; }
int max_prefill_slots() { return 8191; }

}  // namespace kvc
