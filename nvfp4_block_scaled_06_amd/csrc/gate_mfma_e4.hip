// Prefill gate kernels for E <= 64 experts (routing rows of 4 x 16 entries).
#include "gate_mfma.hpp"

namespace nvr {
template hipError_t launch_mma_e<4>(const MmaArgs&, int, int, hipStream_t);
}  // namespace nvr
