// Stand-ins for the kernel launches of libdeltarule, for a host-only build of the C ABI
// (api.cpp and plan.cpp) under the address and undefined-behaviour sanitizers. Every launch
// reports that there is no device; argument validation, planning and the error paths run as in
// the real library.
#include "../../delta_rule_linear_chunked_amd/csrc/common.hpp"
#include "../../delta_rule_linear_chunked_amd/csrc/launch.hpp"

namespace dr {

hipError_t launch_decode(const Params&, int64_t, int, int, bool, bool, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_decode2(const Params&, int64_t, int, int, bool, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_prefill(Params, const PrefillPlan&, void*, int, bool, bool, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_plan_only(Params, const PrefillPlan&, void*, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_backward(BwdParams, int64_t, int, int, bool, bool, hipStream_t) { return hipErrorNoDevice; }
hipError_t scratch_buffer(void**) { return hipErrorNoDevice; }

}  // namespace dr
