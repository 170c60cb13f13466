// Chunked-prefill paged attention (bf16 MFMA).  Placeholder until the
// MFMA kernel lands: reports "not supported".
#include "pa_common.h"

namespace pa {

hipError_t launch_prefill_chunk(const PrefillArgs &, hipStream_t) { return hipErrorNotSupported; }

}  // namespace pa
