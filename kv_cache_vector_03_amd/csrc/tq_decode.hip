// placeholder, replaced below
#include "tq_internal.h"
namespace tq {
DecodePlan plan_decode_unused();
hipError_t launch_decode(const tq_decode_args*, const DecodePlan&, hipStream_t) { return hipErrorNotSupported; }
}
