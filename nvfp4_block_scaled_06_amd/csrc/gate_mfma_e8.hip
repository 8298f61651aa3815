// Prefill gate kernels for E <= 128 experts (routing rows of 8 x 16 entries).
#include "gate_mfma.hpp"

namespace nvr {
template hipError_t launch_mma_e<8>(const MmaArgs&, int, int, hipStream_t);
}  // namespace nvr
