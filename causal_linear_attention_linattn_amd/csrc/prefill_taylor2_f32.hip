// Instantiations of the chunked prefill for one (map, dtype) pair; the
// kernels themselves live in prefill_impl.hpp.
#include "prefill_impl.hpp"

namespace linattn {
#define X(DK, DV) template hipError_t launch_prefill<MAP_TAYLOR2, float, DK, DV, false>(const PrefillArgs&, hipStream_t);
X(16, 16) X(16, 32) X(16, 64)
#undef X
}  // namespace linattn
