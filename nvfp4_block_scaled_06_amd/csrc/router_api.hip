// C ABI of libnvfp4_router.so: argument checks on the host, then launches on
// the caller's stream. No allocation, no host synchronization, no device to
// host copies (commit df05289d, dsv4/layers/grouped_linear.py: caller-owned
// pre-allocated buffers and zero host syncs keep the path capturable).
#include "../../include/nvfp4_router.h"
#include "router_internal.hpp"

#include <algorithm>
#include <mutex>

static_assert(nvr::kScratchOffset == ROUTER_WORKSPACE_STATE_BYTES, "the documented zero-state prefix");

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

size_t gate_need(int64_t T, int64_t D, int64_t E) {
  if (T == 0) return 0;
  const size_t scratch = nvr::gate_scratch_bytes(T, D, E);
  if (nvr::gate_kind(T, D) == nvr::GateKind::kMma && scratch == 0) return 0;  // no counters, no scratch
  return nvr::kScratchOffset + scratch;  // the decode gate needs the regions below kScratchOffset only
}

size_t quantize_need(int64_t rows, int64_t D, bool override_given) {
  const int64_t nblocks = rows * (D / 16);
  // The single-workgroup path needs no scratch; the two-pass path keeps one
  // partial maximum per amax workgroup.
  if (override_given || nblocks <= nvr::kSingleWgMaxBlocks) return 0;
  return nvr::kScratchOffset + nvr::quantize_scratch_bytes();
}

}  // namespace

extern "C" {

size_t router_workspace_bytes(int64_t T, int64_t D, int64_t E, int64_t k) {
  if (!shape_ok(T, D) || E < 1 || E > ROUTER_MAX_EXPERTS || k < 1 || k > E) return 0;
  size_t scratch = nvr::quantize_scratch_bytes();
  const size_t g = nvr::gate_scratch_bytes(T, D, E);
  if (g > scratch) scratch = g;
  if (nvr::batch_fits(T, D)) scratch = std::max(scratch, nvr::batch_scratch_bytes(T, D, E));
  return nvr::kScratchOffset + scratch;
}

int router_workspace_init(void* workspace, size_t bytes, void* stream) {
  if (bytes == 0) return ROUTER_OK;
  if (!workspace || !aligned(workspace, 4) || bytes % 4 != 0) return ROUTER_EINVAL;
  return status_from(nvr::launch_fill_zero(workspace, bytes, static_cast<hipStream_t>(stream)));
}

int router_quantize(const void* x, int64_t rows, int64_t D, const float* gsa_override, uint8_t* codes,
                    uint8_t* scales, float* gsa_out, void* workspace, size_t workspace_bytes, void* stream) {
  if (!shape_ok(rows, D)) return ROUTER_EINVAL;
  if (!gsa_out || (rows > 0 && (!x || !codes || !scales))) return ROUTER_EINVAL;
  if (!aligned(x, 16) || !aligned(codes, 8) || !aligned(gsa_out, 4)) return ROUTER_EINVAL;
  if (gsa_override && !aligned(gsa_override, 4)) return ROUTER_EINVAL;
  const size_t need = quantize_need(rows, D, gsa_override != nullptr);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 256))) return ROUTER_EINVAL;
  void* scratch = need > 0 ? static_cast<char*>(workspace) + nvr::kScratchOffset : nullptr;
  return status_from(nvr::launch_quantize(x, rows, D, gsa_override, codes, scales, gsa_out, scratch,
                                          static_cast<hipStream_t>(stream)));
}

namespace {

int check_gate_args(const uint8_t* x_codes, const uint8_t* x_scales, const float* gsa, const uint8_t* w_codes,
                    const uint8_t* w_scales, const float* gsw, const float* bias, int64_t T, int64_t D, int64_t E,
                    int64_t k, const int32_t* topk_idx, const float* topk_w, const float* logits_out,
                    const void* workspace, size_t workspace_bytes) {
  if (!shape_ok(T, D)) return ROUTER_EINVAL;
  if (E < 1 || k < 1 || k > E) return ROUTER_EINVAL;
  // The gate kernels read K in 32-element chunks (two whole blocks), and the
  // prefill kernel addresses one expert block's weight rows with 32-bit
  // buffer offsets (512 rows of D / 2 bytes stay below 2^31 up to D = 2^22).
  if (E > ROUTER_MAX_EXPERTS || k > ROUTER_MAX_TOPK || D % 32 != 0 || D > ROUTER_MAX_GATE_D)
    return ROUTER_EUNSUPPORTED;
  if (!gsa || !w_codes || !w_scales || !gsw || !bias) return ROUTER_EINVAL;
  if (T > 0 && (!x_codes || !x_scales || !topk_idx || !topk_w)) return ROUTER_EINVAL;
  if (!aligned(x_codes, 16) || !aligned(w_codes, 16) || !aligned(x_scales, 2) || !aligned(w_scales, 2) ||
      !aligned(gsa, 4) || !aligned(gsw, 4) || !aligned(bias, 4) || !aligned(topk_idx, 4) || !aligned(topk_w, 4) ||
      !aligned(logits_out, 4))
    return ROUTER_EINVAL;
  const size_t need = gate_need(T, D, E);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 256))) return ROUTER_EINVAL;
  return ROUTER_OK;
}

}  // namespace

int router_gate_topk(const uint8_t* x_codes, const uint8_t* x_scales, const float* gsa, const uint8_t* w_codes,
                     const uint8_t* w_scales, const float* gsw, const float* bias, float routed_scale, int64_t T,
                     int64_t D, int64_t E, int64_t k, int32_t* topk_idx, float* topk_w, float* logits_out,
                     void* workspace, size_t workspace_bytes, void* stream) {
  const int st = check_gate_args(x_codes, x_scales, gsa, w_codes, w_scales, gsw, bias, T, D, E, k, topk_idx, topk_w,
                                 logits_out, workspace, workspace_bytes);
  if (st != ROUTER_OK) return st;
  const bool ws = gate_need(T, D, E) > 0;
  return status_from(nvr::launch_gate(x_codes, x_scales, gsa, w_codes, w_scales, gsw, bias, routed_scale, T, D, E,
                                      k, topk_idx, topk_w, logits_out, ws ? workspace : nullptr,
                                      static_cast<hipStream_t>(stream)));
}

int router_forward(const void* x, int64_t T, int64_t D, const float* gsa_override, uint8_t* x_codes,
                   uint8_t* x_scales, float* gsa_out, const uint8_t* w_codes, const uint8_t* w_scales,
                   const float* gsw, const float* bias, float routed_scale, int64_t E, int64_t k, int32_t* topk_idx,
                   float* topk_w, float* logits_out, void* workspace, size_t workspace_bytes, void* stream) {
  if (!shape_ok(T, D)) return ROUTER_EINVAL;
  if (!gsa_out || (T > 0 && !x) || !aligned(x, 16) || !aligned(gsa_out, 4) ||
      (gsa_override && !aligned(gsa_override, 4)))
    return ROUTER_EINVAL;
  int st = check_gate_args(x_codes, x_scales, gsa_out, w_codes, w_scales, gsw, bias, T, D, E, k, topk_idx, topk_w,
                           logits_out, workspace, workspace_bytes);
  if (st != ROUTER_OK) return st;
  const size_t qneed = quantize_need(T, D, gsa_override != nullptr);
  if (qneed > 0 && (!workspace || workspace_bytes < qneed || !aligned(workspace, 256))) return ROUTER_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(workspace);
  if (T > 0 && nvr::batch_fits(T, D)) {
    const size_t need = nvr::kScratchOffset + nvr::batch_scratch_bytes(T, D, E);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 256)) return ROUTER_EINVAL;
    return status_from(nvr::launch_forward_batch(x, gsa_override, x_codes, x_scales, gsa_out, w_codes, w_scales, gsw,
                                                 bias, routed_scale, T, D, E, k, topk_idx, topk_w, logits_out,
                                                 base + nvr::kScratchOffset, s));
  }
  if (T > 0 && nvr::forward_single_launch(T, D)) {
    return status_from(nvr::launch_forward_fused(x, gsa_override, x_codes, x_scales, gsa_out, w_codes, w_scales, gsw,
                                                 bias, routed_scale, T, D, E, k, topk_idx, topk_w, logits_out, base,
                                                 s));
  }
  // Larger T: the quantize kernels then the gate kernels, back to back on the stream.
  hipError_t err = nvr::launch_quantize(x, T, D, gsa_override, x_codes, x_scales, gsa_out,
                                        qneed > 0 ? base + nvr::kScratchOffset : nullptr, s);
  if (err != hipSuccess) return ROUTER_EHIP;
  const bool ws = gate_need(T, D, E) > 0;
  return status_from(nvr::launch_gate(x_codes, x_scales, gsa_out, w_codes, w_scales, gsw, bias, routed_scale, T, D,
                                      E, k, topk_idx, topk_w, logits_out, ws ? workspace : nullptr, s));
}

const char* router_status_string(int status) {
  switch (status) {
    case ROUTER_OK: return "ok";
    case ROUTER_EINVAL: return "invalid argument (shape, null or misaligned pointer, or workspace too small)";
    case ROUTER_EUNSUPPORTED: return "unsupported size (E > 512, k > 32, or a gate call with D % 32 != 0 or D > 2^22)";
    case ROUTER_EHIP: return "HIP launch error";
    case ROUTER_ESCRATCH:
      return "the call needs more scratch than the library's static buffer holds (ROUTER_STATIC_SCRATCH_BYTES = "
             "16 MiB); use router_forward with a workspace";
    default: return "unknown status";
  }
}

}  // extern "C"

// ---------------------------------------------------------------------------
// router_forward_noalloc: router_forward with the library's own scratch, for
// callers that cannot allocate. The scratch is one static device array per
// GPU (it lives as long as the process). Host code never passes the array's
// name to a kernel: `scratch` names a host-side stand-in there. Its device
// address comes from hipGetSymbolAddress, once per device, and only that
// address is used.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[ROUTER_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of the current device's `scratch`, set up on its first
// use: the symbol's address, then one clear of the part every call expects
// zero between calls (the counters and the decode region; static storage
// starts zeroed, and every call leaves them zero, so this clear only makes
// that state explicit). The clear is a kernel on the caller's stream, ordered
// before the call it precedes.
int static_scratch(void** out, hipStream_t stream) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ROUTER_EHIP;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return ROUTER_EHIP;
    if (nvr::launch_fill_zero(p, nvr::kScratchOffset, stream) != hipSuccess) return ROUTER_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ROUTER_OK;
}

}  // namespace

extern "C" int router_forward_noalloc(const void* x, int64_t T, int64_t D, const float* gsa_override,
                                      uint8_t* x_codes, uint8_t* x_scales, float* gsa_out, const uint8_t* w_codes,
                                      const uint8_t* w_scales, const float* gsw, const float* bias,
                                      float routed_scale, int64_t E, int64_t k, int32_t* topk_idx, float* topk_w,
                                      float* logits_out, void* stream) {
  const size_t need = router_workspace_bytes(T, D, E, k);
  if (need == 0) {  // invalid or unsupported sizes: router_forward says which, before any launch
    return router_forward(x, T, D, gsa_override, x_codes, x_scales, gsa_out, w_codes, w_scales, gsw, bias,
                          routed_scale, E, k, topk_idx, topk_w, logits_out, nullptr, 0, stream);
  }
  if (need > ROUTER_STATIC_SCRATCH_BYTES) return ROUTER_ESCRATCH;
  void* ws = nullptr;
  const int st = static_scratch(&ws, static_cast<hipStream_t>(stream));
  if (st != ROUTER_OK) return st;
  return router_forward(x, T, D, gsa_override, x_codes, x_scales, gsa_out, w_codes, w_scales, gsw, bias,
                        routed_scale, E, k, topk_idx, topk_w, logits_out, ws, ROUTER_STATIC_SCRATCH_BYTES, stream);
}
