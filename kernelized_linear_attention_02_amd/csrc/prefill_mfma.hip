// bf16 matrix-core prefill (d_qk = d_v = 64). Not enabled yet: the generic
// float32 path serves every shape until this kernel passes parity.
#include "kla_device.hpp"
#include "kla_internal.hpp"

namespace kla {

bool prefill_mfma_supported(const PrefillArgs&) { return false; }
size_t prefill_mfma_workspace(const PrefillArgs&) { return 0; }
hipError_t prefill_mfma_launch(const PrefillArgs&, void*, hipStream_t) { return hipErrorNotSupported; }

}  // namespace kla
