// Prefill-route kernels (placeholder translation unit; filled in below).
#include "msa_common.h"
#include "msa_kernels.h"

namespace msa {}  // namespace msa
