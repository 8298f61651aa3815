// Prefill gate kernels for E <= 256 experts (routing rows of 16 x 16 entries).
#include "gate_mfma.hpp"

namespace nvr {
template hipError_t launch_mma_e<16>(const MmaArgs&, int, int, hipStream_t);
}  // namespace nvr
