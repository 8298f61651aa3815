// C ABI of libnvfp4_router.so: argument checks on the host, then launches on
// the caller's stream. No allocation, no host synchronization, no device to
// host copies (commit df05289d, dsv4/layers/grouped_linear.py: caller-owned
// pre-allocated buffers and zero host syncs keep the path capturable).
#include "../../include/nvfp4_router.h"
#include "router_internal.hpp"

namespace {

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Bounds that keep every element count and byte offset far inside int64 and
// every grid dimension inside int32.
constexpr int64_t kMaxD = int64_t(1) << 24;
constexpr int64_t kMaxRows = int64_t(1) << 31;
constexpr int64_t kMaxElems = int64_t(1) << 40;

bool shape_ok(int64_t rows, int64_t D) {
  return rows >= 0 && rows < kMaxRows && D >= 16 && D <= kMaxD && D % 16 == 0 && rows * D <= kMaxElems;
}

int status_from(hipError_t e) { return e == hipSuccess ? ROUTER_OK : ROUTER_EHIP; }

size_t quantize_need(int64_t rows, int64_t D, bool override_given) {
  const int64_t nblocks = rows * (D / 16);
  // The single-workgroup path needs no scratch; the two-pass path keeps one
  // partial maximum per amax workgroup.
  if (override_given || nblocks <= nvr::kSingleWgMaxBlocks) return 0;
  return nvr::kCounterBytes + nvr::quantize_scratch_bytes();
}

}  // namespace

extern "C" {

size_t router_workspace_bytes(int64_t T, int64_t D, int64_t E, int64_t k) {
  if (!shape_ok(T, D) || E < 1 || E > ROUTER_MAX_EXPERTS || k < 1 || k > E) return 0;
  size_t scratch = nvr::quantize_scratch_bytes();
  const size_t g = nvr::gate_scratch_bytes(T, D, E);
  if (g > scratch) scratch = g;
  return nvr::kCounterBytes + scratch;
}

int router_workspace_init(void* workspace, size_t bytes, void* stream) {
  if (bytes == 0) return ROUTER_OK;
  if (!workspace || !aligned(workspace, 4) || bytes % 4 != 0) return ROUTER_EINVAL;
  return status_from(nvr::launch_fill_zero(workspace, bytes, static_cast<hipStream_t>(stream)));
}

int router_quantize(const void* x, int64_t rows, int64_t D, const float* gsa_override, uint8_t* codes,
                    uint8_t* scales, float* gsa_out, void* workspace, size_t workspace_bytes, void* stream) {
  if (!shape_ok(rows, D)) return ROUTER_EINVAL;
  if (!x || !codes || !scales || !gsa_out) return ROUTER_EINVAL;
  if (!aligned(x, 16) || !aligned(codes, 8) || !aligned(gsa_out, 4)) return ROUTER_EINVAL;
  if (gsa_override && !aligned(gsa_override, 4)) return ROUTER_EINVAL;
  const size_t need = quantize_need(rows, D, gsa_override != nullptr);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 256))) return ROUTER_EINVAL;
  void* scratch = need > 0 ? static_cast<char*>(workspace) + nvr::kCounterBytes : nullptr;
  return status_from(nvr::launch_quantize(x, rows, D, gsa_override, codes, scales, gsa_out, scratch,
                                          static_cast<hipStream_t>(stream)));
}

int router_gate_topk(const uint8_t* x_codes, const uint8_t* x_scales, const float* gsa, const uint8_t* w_codes,
                     const uint8_t* w_scales, const float* gsw, const float* bias, float routed_scale, int64_t T,
                     int64_t D, int64_t E, int64_t k, int32_t* topk_idx, float* topk_w, float* logits_out,
                     void* workspace, size_t workspace_bytes, void* stream) {
  if (!shape_ok(T, D) || D % 32 != 0) return ROUTER_EINVAL;
  if (E < 1 || k < 1 || k > E) return ROUTER_EINVAL;
  if (E > ROUTER_MAX_EXPERTS || k > ROUTER_MAX_TOPK) return ROUTER_EUNSUPPORTED;
  if (!x_codes || !x_scales || !gsa || !w_codes || !w_scales || !gsw || !bias || !topk_idx || !topk_w)
    return ROUTER_EINVAL;
  if (!aligned(x_codes, 16) || !aligned(w_codes, 16) || !aligned(x_scales, 2) || !aligned(w_scales, 2) ||
      !aligned(gsa, 4) || !aligned(gsw, 4) || !aligned(bias, 4) || !aligned(topk_idx, 4) || !aligned(topk_w, 4) ||
      (logits_out && !aligned(logits_out, 4)))
    return ROUTER_EINVAL;
  size_t need = 0;
  if (T > 0 && nvr::use_split_gate(T)) need = nvr::kCounterBytes + nvr::gate_scratch_bytes(T, D, E);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 256))) return ROUTER_EINVAL;
  uint32_t* counters = need > 0 ? static_cast<uint32_t*>(workspace) : nullptr;
  void* scratch = need > 0 ? static_cast<char*>(workspace) + nvr::kCounterBytes : nullptr;
  return status_from(nvr::launch_gate(x_codes, x_scales, gsa, w_codes, w_scales, gsw, bias, routed_scale, T, D, E,
                                      k, topk_idx, topk_w, logits_out, counters, scratch,
                                      static_cast<hipStream_t>(stream)));
}

const char* router_status_string(int status) {
  switch (status) {
    case ROUTER_OK: return "ok";
    case ROUTER_EINVAL: return "invalid argument (shape, null or misaligned pointer, or workspace too small)";
    case ROUTER_EUNSUPPORTED: return "unsupported size (E > 512 or k > 32)";
    case ROUTER_EHIP: return "HIP launch error";
    default: return "unknown status";
  }
}

}  // extern "C"
