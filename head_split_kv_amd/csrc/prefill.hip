// Chunked-prefill attention (placeholder until the MFMA kernel lands).
#include <hip/hip_runtime.h>

#include "duo_internal.h"

namespace duo {
int launch_prefill(const PrefillArgs&, int, int, int, void*) { return -1; }
}  // namespace duo
