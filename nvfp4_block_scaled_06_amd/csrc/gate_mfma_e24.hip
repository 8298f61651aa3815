// Prefill gate kernels for E <= 384 experts (routing rows of 24 x 16 entries).
#include "gate_mfma.hpp"

namespace nvr {
template hipError_t launch_mma_e<24>(const MmaArgs&, int, int, hipStream_t);
}  // namespace nvr
