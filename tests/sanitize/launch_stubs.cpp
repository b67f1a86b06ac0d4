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
// the chunked backward's record: d_k x d_k operand fragments (4 bytes per element) and d_k x d_v fp32
int64_t cbwd_record_bytes(int dk, int dv) { return ((int64_t)dk * dk * 4 + (int64_t)dk * dv * 4 + 255) / 256 * 256; }
hipError_t launch_chunked_backward(const CbParams&, int, bool, bool, hipStream_t) { return hipErrorNoDevice; }

}  // namespace dr
