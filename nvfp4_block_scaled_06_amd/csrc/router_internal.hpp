// Internal launch interface between the C-ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nvr {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Workspace layout: [0, kCounterBytes) arrival counters of the split gate
// (zero between calls); [kCounterBytes, ...) per-call scratch (partial
// maxima of the quantizer, partial logits of the split gate).
constexpr size_t kCounterBytes = 256;
constexpr int kMaxCounters = (int)(kCounterBytes / sizeof(uint32_t));

constexpr int kSingleWgMaxBlocks = 2048;  // single-workgroup quantizer up to this many blocks
constexpr int kAmaxPartials = 1024;       // workgroups of the amax pass
constexpr int kQuantMaxGrid = 8192;  // workgroups of the quantize pass

// Gate dispatch: T <= split_max_t uses the split gate (experts x K split over
// many workgroups, arrival counter, the last workgroup of a 16-row tile runs
// the epilogue); larger T uses the fused gate (one workgroup per 32 rows and
// all experts, epilogue in the same workgroup).
struct GateTuning {
  int split_max_t = 256;
  int split_target_wgs = 128;
  int split_max_ksplit = 64;
};
const GateTuning& gate_tuning();

struct SplitPlan {
  int col_groups;  // workgroups along experts (4 waves x 16 experts each)
  int row_tiles;   // 16-row tiles
  int ksplit;      // K ranges
  int nsteps;      // 128-element K steps in D
};
SplitPlan plan_split(int64_t T, int64_t D, int64_t E);
bool use_split_gate(int64_t T);

size_t quantize_scratch_bytes();
size_t gate_scratch_bytes(int64_t T, int64_t D, int64_t E);

hipError_t launch_quantize(const void* x, int64_t rows, int64_t D, const float* gsa_override, uint8_t* codes,
                           uint8_t* scales, float* gsa_out, void* scratch, hipStream_t stream);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t stream);
hipError_t launch_gate(const uint8_t* x_codes, const uint8_t* x_scales, const float* gsa, const uint8_t* w_codes,
                       const uint8_t* w_scales, const float* gsw, const float* bias, float routed_scale, int64_t T,
                       int64_t D, int64_t E, int64_t k, int32_t* topk_idx, float* topk_w, float* logits_out,
                       uint32_t* counters, void* scratch, hipStream_t stream);

}  // namespace nvr
