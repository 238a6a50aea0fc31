// Instantiations of the gated (scalar-decay) chunked prefill for one
// (map, dtype) pair; the kernels themselves live in prefill_impl.hpp.
#include "prefill_impl.hpp"

namespace linattn {
#define X(DK, DV) template hipError_t launch_prefill<MAP_TAYLOR2, bf16_t, DK, DV, true>(const PrefillArgs&, hipStream_t);
X(16, 16) X(16, 32) X(16, 64)
#undef X
}  // namespace linattn
