// Matrix-core (MFMA) decode kernel for query groups of 16 or 32 rows per kv head.
#include "pa_internal.h"

namespace pa {

bool mfma_supported(const pa_dims&) { return false; }

hipError_t launch_decode_mfma(const DecodeParams&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace pa
