// Decode (S = 1) specialisation: not yet specialised; chunk_len == 1 runs the
// general chunk kernels, which need no workspace.
#include "h2o_internal.h"

namespace h2o {

size_t decode_workspace_bytes(int, int, int, int) { return 0; }

hipError_t launch_decode(const ChunkArgs&, void*, hipStream_t) { return hipErrorNotSupported; }

}  // namespace h2o
