// Varlen causal prefill attention, bf16 storage, head_dim 128, on gfx950 MFMA.
#include "common.h"
#include "launch.h"

namespace pkv {

bool prefill_fast_supported(int, int, bool) { return false; }

hipError_t launch_prefill_bf16(const AttnArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace pkv
