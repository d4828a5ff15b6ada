#include "prefill.h"

namespace moe {

bool prefill_supported(const moe_config&) { return false; }
moe_status prefill_forward(void**, const PrefillArgs&, hipStream_t) { return MOE_EINVAL; }
void prefill_free(void*) {}

}  // namespace moe
