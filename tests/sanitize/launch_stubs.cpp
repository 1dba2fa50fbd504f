// Device entry points of the library replaced by stubs, for a host-only build of
// kvq_api.cpp and kvq_stream.cpp under the host sanitizers (no GPU code is built).
// Every stub reports that no device is present, as the real library does on a
// machine without a GPU, so validation runs exactly as in the real build.
#include <hip/hip_runtime.h>

#include "kvq_internal.hpp"

namespace kvq {

hipError_t launch_side_pack(const SideArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_pack(const PackArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_append(const AppendArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_read_probe(const void*, size_t, uint32_t*, hipStream_t) { return hipErrorNoDevice; }
hipError_t static_scratch(void**) { return hipErrorNoDevice; }
hipError_t device_cus(int*, int*) { return hipErrorNoDevice; }
bool mfma_takes(const kvq_layout&, int) { return false; }
hipError_t mfma_decode(const DecodeArgs&, hipStream_t, DecodePlan*, bool) { return hipErrorNoDevice; }
hipError_t plan_decode(const DecodeArgs&, DecodePlan*) { return hipErrorNoDevice; }
hipError_t launch_decode(const DecodeArgs&, const DecodePlan&, hipStream_t, hipEvent_t) { return hipErrorNoDevice; }

}  // namespace kvq
