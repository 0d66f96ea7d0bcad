// Chunk-32 MFMA KDA prefill for gfx950 (placeholder until the kernel lands).
#include "kda_internal.h"

namespace kda {

hipError_t launch_prefill_chunk(const PrefillArgs&, int, int, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace kda
