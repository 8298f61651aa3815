// Prefill gate kernels for E <= 512 experts (routing rows of 32 x 16 entries).
#include "gate_mfma.hpp"

namespace nvr {
template hipError_t launch_mma_e<32>(const MmaArgs&, int, int, hipStream_t);
}  // namespace nvr
