// Chunked VLA forward (time-segment parallel).  Not built yet: every query reports the
// path as unsupported, so VLA_PATH_AUTO resolves to the sequential path.
#include "vla_internal.h"

namespace vla {

int chunk_default(const Problem &) { return 64; }
bool chunk_supported(const Problem &, int) { return false; }
size_t chunk_workspace_bytes(const Problem &, int) { return 0; }
hipError_t launch_chunk(const Problem &, int, const void *, const void *, const void *,
                        const void *, void *, float *, float *, void *, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace vla
