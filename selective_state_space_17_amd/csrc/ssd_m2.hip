// Mamba-2 scalar-A multi-head (SSD) form -- placeholder until the matrix-core kernel lands.
#include "internal.h"

namespace mssm {

size_t ssd_workspace_bytes(int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, int64_t) { return 0; }

hipError_t ssd_launch(const SSDArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace mssm
