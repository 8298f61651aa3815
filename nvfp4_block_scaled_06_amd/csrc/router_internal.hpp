// Internal launch interface between the C-ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nvr {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Workspace layout:
//   [0, kCounterBytes)     arrival counters of the tile and split-expert
//                          gates and the lm_head: zero between calls (every
//                          call that counts returns its counter to zero);
//   [kDecodeRegionOffset, kScratchOffset)
//                          the decode gate's flagged slice partials: zero
//                          between calls (the call that writes a word also
//                          clears it), and written by no other kernel;
//   [kScratchOffset, ...)  per-call scratch (partial maxima of the quantizer,
//                          the [T, E] logits of the tile gate and of the
//                          split-expert prefill gate, the batched-decode
//                          forward's partial maxima and flagged slice
//                          partials, the lm_head's per-workgroup candidates).
constexpr size_t kCounterBytes = 4096;
constexpr int kMaxCounters = (int)(kCounterBytes / sizeof(uint32_t));
constexpr size_t kDecodeRegionOffset = kCounterBytes;
constexpr size_t kDecodeRegionBytes = 128 * 1024;
constexpr size_t kScratchOffset = kDecodeRegionOffset + kDecodeRegionBytes;

constexpr int kSingleWgMaxBlocks = 2048;  // single-workgroup quantizer up to this many blocks
constexpr int kAmaxPartials = 1024;       // workgroups of the amax pass
constexpr int kQuantMaxGrid = 8192;  // workgroups of the quantize pass

// Gate dispatch by token count: decode (T <= 4 and D <= 16384: one workgroup
// per 16 experts and 1024-element K slice, the last workgroup routes), tile
// (T <= split_max_t: 16x16 MFMA tiles, the last workgroup of each 16-row tile
// routes), mfma (larger T: BM tokens x 128 NTW experts per workgroup on
// 32x32 MFMA; routed in the workgroup, or by the last expert block of each
// token block when E is split).
struct GateTuning {
  int split_max_t = 256;
  int mma_bm = 0;   // prefill tokens per workgroup (32 / 64 / 128); 0 = planned
  int mma_ntw = 0;  // prefill 32-expert tiles per wavefront; 0 = planned
};
const GateTuning& gate_tuning();

enum class GateKind { kDecode, kTile, kMma };
GateKind gate_kind(int64_t T, int64_t D);

size_t quantize_scratch_bytes();
size_t gate_scratch_bytes(int64_t T, int64_t D, int64_t E);

hipError_t launch_quantize(const void* x, int64_t rows, int64_t D, const float* gsa_override, uint8_t* codes,
                           uint8_t* scales, float* gsa_out, void* scratch, hipStream_t stream);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t stream);
hipError_t launch_gate(const uint8_t* x_codes, const uint8_t* x_scales, const float* gsa, const uint8_t* w_codes,
                       const uint8_t* w_scales, const float* gsw, const float* bias, float routed_scale, int64_t T,
                       int64_t D, int64_t E, int64_t k, int32_t* topk_idx, float* topk_w, float* logits_out,
                       void* workspace, hipStream_t stream);

// Decode-size gate (gate_decode.hip): whether T x D takes it, and its launch
// (reading quantized x). It uses the workspace's decode region only.
bool decode_fits(int64_t T, int64_t D);
hipError_t launch_decode_gate(const uint8_t* x_codes, const uint8_t* x_scales, const float* gsa,
                              const uint8_t* w_codes, const uint8_t* w_scales, const float* gsw, const float* bias,
                              float routed_scale, int64_t T, int64_t D, int64_t E, int64_t k, int32_t* topk_idx,
                              float* topk_w, float* logits_out, void* workspace, hipStream_t stream);

// Quantize + gate in one launch (decode-size T only; see forward_single_launch).
bool forward_single_launch(int64_t T, int64_t D);
hipError_t launch_forward_fused(const void* x, const float* gsa_override, uint8_t* x_codes, uint8_t* x_scales,
                                float* gsa_out, const uint8_t* w_codes, const uint8_t* w_scales, const float* gsw,
                                const float* bias, float routed_scale, int64_t T, int64_t D, int64_t E, int64_t k,
                                int32_t* topk_idx, float* topk_w, float* logits_out, void* workspace,
                                hipStream_t stream);

// Batched-decode forward (gate_batch.hip; router_forward only): 4 < T <= 256
// and D <= 16384, in two launches. Its per-call scratch (partial maxima, then
// the flagged slice partials, batch_scratch_bytes in all) starts at
// kScratchOffset.
bool batch_fits(int64_t T, int64_t D);
size_t batch_scratch_bytes(int64_t T, int64_t D, int64_t E);
hipError_t launch_forward_batch(const void* x, const float* gsa_override, uint8_t* x_codes, uint8_t* x_scales,
                                float* gsa_out, const uint8_t* w_codes, const uint8_t* w_scales, const float* gsw,
                                const float* bias, float routed_scale, int64_t T, int64_t D, int64_t E, int64_t k,
                                int32_t* topk_idx, float* topk_w, float* logits_out, void* scratch,
                                hipStream_t stream);

}  // namespace nvr
