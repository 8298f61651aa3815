/*
 * nvfp4_router.h -- C ABI of the MI355X (gfx950) NVFP4 dense-MoE router library
 * (libnvfp4_router.so).
 *
 * The path: runtime NVFP4 quantization of the activations, the block-scaled
 * gate projection to per-expert logits, and the fused six-step routing
 * epilogue. Sources are three commit pages of the nvfp4-megamoe-kernel
 * repository:
 *   - commit 04cf8ca8, dsv4/layers/router.py: runtime global scale
 *     gsa = max|x| / (6 * 448), the E4M3 block-scale ceiling of 448, the
 *     NVFP4 gate GEMM and the fused-router dispatch order;
 *   - commit e0f60b9f, dsv4/kernels/router/__init__.py: the six-step
 *     single-pass activation/top-k epilogue after the gate GEMM;
 *   - commit df05289d, dsv4/layers/grouped_linear.py: one flattened
 *     quantize launch with a device-only global scale, no host syncs and
 *     caller-owned pre-allocated buffers.
 * The NVFP4 format fixes the rest: 16-element blocks along the contraction
 * axis, E4M3 (OCP "FN", max 448) block scales, E2M1 element codes, one fp32
 * per-tensor global scale.
 *
 * Conventions shared by every entry point:
 *   - Every tensor pointer is a DEVICE pointer owned by the caller; tensors
 *     are dense and row-major. The library allocates nothing and keeps no
 *     per-call state; it only enqueues work on `stream` (a hipStream_t, NULL
 *     for the default stream) and never synchronizes or copies to the host,
 *     so calls may be captured in a HIP graph.
 *   - A negative return value means the arguments were rejected on the host
 *     and nothing was enqueued, except ROUTER_EHIP (a launch failed).
 *   - Data pointers of an empty batch (rows or T == 0) may be NULL; the
 *     global scale output is still written (0, or the override).
 *   - Non-finite input values are a precondition violation: they make the
 *     global scale non-finite (the device-visible error flag) and leave the
 *     other outputs unspecified.
 *   - Calls that share one workspace must not overlap in time (enqueue them
 *     on one stream).
 *   - Tuning overrides, read once per process from the environment (results
 *     stay within the stated tolerances for any accepted value; invalid
 *     values are ignored): NVR_SPLIT_MAX_T (largest T on the 16x16-tile
 *     gate, default 256), NVR_MMA_BM (prefill tokens per workgroup: 32, 64
 *     or 128) with NVR_MMA_NTW (32-expert tiles per wavefront, 1..4). The
 *     workspace size follows the same settings, so set them before the first
 *     call and leave them.
 */
#ifndef NVFP4_ROUTER_H
#define NVFP4_ROUTER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ROUTER_OK 0
#define ROUTER_EINVAL (-1)       /* bad shape, null or misaligned pointer, workspace too small */
#define ROUTER_EUNSUPPORTED (-2) /* a documented size limit is exceeded */
#define ROUTER_EHIP (-3)         /* a kernel launch reported an error */
#define ROUTER_ESCRATCH (-4)     /* router_forward_noalloc: the call needs more than the static scratch */

#define ROUTER_MAX_EXPERTS 512
#define ROUTER_MAX_TOPK 32
#define ROUTER_MAX_GATE_D (1 << 22) /* largest hidden size of a gate call */
#define ROUTER_STATIC_SCRATCH_BYTES (16 << 20) /* router_forward_noalloc's scratch, per GPU */
#define ROUTER_WORKSPACE_STATE_BYTES (4096 + 131072) /* workspace prefix that stays zero between calls */

/*
 * Bytes of workspace that router_quantize and router_gate_topk need for a
 * call with these sizes (rows = T tokens, D hidden, E experts, k chosen).
 * One workspace sized by this function serves both calls. The caller
 * allocates it once, ahead of time, and reuses it for every call, so that no
 * call allocates or synchronizes and a decode loop can be captured in a
 * graph (commit df05289d, dsv4/layers/grouped_linear.py: the fixes that
 * pre-allocate the output buffer and the expert-offset range buffer once at
 * initialization instead of per call).
 *
 * The first ROUTER_WORKSPACE_STATE_BYTES bytes (arrival counters, then the
 * decode gate's flagged partials) must be zero before the first call
 * (allocate zero-filled memory or call router_workspace_init), and every call
 * leaves them zero again; the rest is per-call scratch. Every size this
 * function returns covers that state. Calls that share one workspace must be
 * ordered (one stream); concurrent calls need workspaces of their own.
 * Returns 0 for invalid sizes.
 */
size_t router_workspace_bytes(int64_t T, int64_t D, int64_t E, int64_t k);

/*
 * Zero-fills `bytes` of `workspace` on `stream` with a kernel (no memset
 * node, so it may be captured). Needed once per workspace allocation, at the
 * same initialization time as the allocation itself (the pre-allocated
 * buffers of commit df05289d, dsv4/layers/grouped_linear.py).
 * ROUTER_EINVAL if `workspace` is NULL or not 4-byte aligned, or `bytes` is
 * not a multiple of 4 (bytes == 0 does nothing).
 */
int router_workspace_init(void* workspace, size_t bytes, void* stream);

/*
 * Runtime NVFP4 quantization of x (the flattened single-launch quantizer
 * with a device-only global scale: commit df05289d,
 * dsv4/layers/grouped_linear.py; the scale rule: commit 04cf8ca8,
 * dsv4/layers/router.py, runtime-gsa paragraph).
 *
 *   x            [rows, D] bf16 bit patterns, 16-byte aligned.
 *   rows, D      rows >= 0, D >= 16, D % 16 == 0.
 *   gsa_override NULL: gsa = fp32(max|x|) / 2688 (one IEEE fp32 division).
 *                Else a device fp32 scalar used as gsa instead (reproduces a
 *                static scale; must be >= 0 and finite).
 *   codes        [rows, D/2] out: E2M1 codes, element 2i in the low nibble of
 *                byte i; each code is the E2M1 value nearest to
 *                |x| / (gsa * S) (ties to even, saturating at 6) with the
 *                sign bit of x. 8-byte aligned.
 *   scales       [rows, D/16] out: E4M3FN bytes; each is the E4M3 value nearest
 *                to bmax / (6 * gsa) over its 16-element block (ties to even,
 *                saturating at 448).
 *   gsa_out      [1] out: the global scale used (device fp32).
 * gsa == 0 gives zero scale bytes and sign-only codes. Every rounding is
 * exact (identical to the infinitely precise quotient's).
 *
 * Also used at load time on bf16 gate weights [E, D] (their gsa is gsw).
 */
int router_quantize(const void* x, int64_t rows, int64_t D, const float* gsa_override, uint8_t* codes,
                    uint8_t* scales, float* gsa_out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Gate projection plus the fused routing epilogue (gate GEMM on NVFP4
 * operands: commit 04cf8ca8, dsv4/layers/router.py; six-step epilogue:
 * commit e0f60b9f, dsv4/kernels/router/__init__.py).
 *
 *   x_codes, x_scales, gsa   router_quantize outputs for x [T, D].
 *   w_codes, w_scales, gsw   the gate weights in the same format, [E, D/2],
 *                            [E, D/16] and a device fp32 scalar.
 *   bias                     [E] fp32 selection bias.
 *   routed_scale             host fp32 factor applied after renormalization.
 *   T, D, E, k               T >= 0; 1 <= k <= E; D >= 16, D % 16 == 0
 *                            (ROUTER_EINVAL otherwise). The gate kernels
 *                            read K in 32-element chunks, so D % 32 != 0,
 *                            D > ROUTER_MAX_GATE_D, E > 512 and k > 32 give
 *                            ROUTER_EUNSUPPORTED.
 *   topk_idx                 [T, k] int32 out: experts by descending
 *                            s + bias, an exact tie going to the lower index.
 *   topk_w                   [T, k] fp32 out: routed_scale * s / sum(s) over
 *                            the chosen experts, s = sigmoid(logit).
 *   logits_out               NULL, or [T, E] fp32 out: the logits
 *                            gsa * gsw * sum_d xhat * what (fp32 accumulation).
 * Code and scale pointers must be 16- and 2-byte aligned.
 */
int router_gate_topk(const uint8_t* x_codes, const uint8_t* x_scales, const float* gsa, const uint8_t* w_codes,
                     const uint8_t* w_scales, const float* gsw, const float* bias, float routed_scale, int64_t T,
                     int64_t D, int64_t E, int64_t k, int32_t* topk_idx, float* topk_w, float* logits_out,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * router_quantize followed by router_gate_topk, in one call and with the same
 * results: x_codes, x_scales and gsa_out are written exactly as
 * router_quantize writes them, and the routing is that of router_gate_topk on
 * them. For decode-size batches (T <= 4, D <= 16384) it is a single kernel
 * launch (the single-launch fused router that commit 04cf8ca8,
 * dsv4/layers/router.py, gives priority over the two-launch path): every
 * workgroup derives gsa from all of x and quantizes the blocks it multiplies
 * in registers. Batched decode (4 < T <= 256, D <= 16384) is two launches: a
 * pass that takes the partial maxima of x, then one kernel that quantizes,
 * multiplies and routes (each workgroup quantizes the x tile it multiplies).
 * Larger T runs the quantize kernels and then the gate kernels.
 *
 * Arguments as in the two calls above: x [T, D] bf16 (16-byte aligned);
 * x_codes (16-byte aligned), x_scales and gsa_out are outputs; the size
 * limits of router_gate_topk apply (ROUTER_EUNSUPPORTED beyond them).
 * The workspace must satisfy router_workspace_bytes(T, D, E, k).
 */
int router_forward(const void* x, int64_t T, int64_t D, const float* gsa_override, uint8_t* x_codes,
                   uint8_t* x_scales, float* gsa_out, const uint8_t* w_codes, const uint8_t* w_scales,
                   const float* gsw, const float* bias, float routed_scale, int64_t E, int64_t k, int32_t* topk_idx,
                   float* topk_w, float* logits_out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * router_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). It takes the same arguments as
 * router_forward minus the workspace and gives the same results from the same
 * kernels. Its scratch is a static device array of
 * ROUTER_STATIC_SCRATCH_BYTES (16 MiB) that each GPU the library runs on
 * holds until the process ends; the call itself allocates nothing and calls
 * no allocating routine. The first call on a device looks up that array's
 * address and enqueues one clear of its counters on `stream`.
 *
 * Calls whose router_workspace_bytes(T, D, E, k) exceeds 16 MiB (prefill
 * batches whose experts are split over workgroups with T * E * 4 above it,
 * e.g. T = 16384 at E = 256; batched-decode calls whose slice partials,
 * 4 * T * E * ceil(D / 256) bytes, exceed it, e.g. T = 256, D = 16384,
 * E = 512) return ROUTER_ESCRATCH before any launch;
 * invalid or unsupported sizes give router_forward's status. Every call on one
 * GPU shares that GPU's array: calls that overlap in time on one GPU (other
 * streams, other threads) race and give wrong results; enqueue them in order.
 */
int router_forward_noalloc(const void* x, int64_t T, int64_t D, const float* gsa_override, uint8_t* x_codes,
                           uint8_t* x_scales, float* gsa_out, const uint8_t* w_codes, const uint8_t* w_scales,
                           const float* gsw, const float* bias, float routed_scale, int64_t E, int64_t k,
                           int32_t* topk_idx, float* topk_w, float* logits_out, void* stream);

/*
 * Static text for a status code. The library reports every rejection as a
 * return value and never synchronizes to report one (the zero-host-sync rule
 * of commit df05289d, dsv4/layers/grouped_linear.py); this turns the value
 * into a message. Unknown codes give "unknown status".
 */
const char* router_status_string(int status);

/*
 * lm_head-shaped NVFP4 GEMV with a greedy (top-1) epilogue: for each of T
 * tokens, logits[t, n] = gsa * gsw * sum_d xhat[t, d] * what[n, d] (fp32
 * accumulation, the same arithmetic as the router's gate) over an N-row
 * vocabulary matrix, and the row with the largest logit (an exact tie going
 * to the lower row). The NVFP4 lm_head replaces a 1.8 GB BF16 weight (commit
 * df05289d, dsv4/layers/grouped_linear.py, weights paragraph); at decode
 * size the call streams the packed weights once.
 *
 *   x_codes, x_scales, gsa   router_quantize outputs for x [T, D] (16- and
 *                            2-byte aligned).
 *   w_codes, w_scales, gsw   the weights in the same format: [N, D/2],
 *                            [N, D/16] (16- and 2-byte aligned) and a device
 *                            fp32 scalar.
 *   T, D, N                  0 <= T <= 4; 32 <= D <= 16384, D % 32 == 0;
 *                            T * D <= 32768; 1 <= N <= 2^30.
 *   out_idx, out_logit       [T] int32 / fp32 out: the chosen row and its
 *                            logit.
 *   logits_out               NULL, or [T, N] fp32 out: every logit.
 *   workspace                256-byte aligned, lmhead_workspace_bytes(T, D,
 *                            N) bytes; its first
 *                            ROUTER_WORKSPACE_STATE_BYTES bytes are the state
 *                            shared with the router calls (zero between
 *                            calls, see router_workspace_bytes).
 * Returns ROUTER_EINVAL for bad shapes, pointers or workspace.
 */
size_t lmhead_workspace_bytes(int64_t T, int64_t D, int64_t N);
int lmhead_argmax(const uint8_t* x_codes, const uint8_t* x_scales, const float* gsa, const uint8_t* w_codes,
                  const uint8_t* w_scales, const float* gsw, int64_t T, int64_t D, int64_t N, int32_t* out_idx,
                  float* out_logit, float* logits_out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Group offsets of the grouped linear layer, on the device: offsets[g] =
 * range[g] * padded_rows for g = 0 .. G (G + 1 values), group g owning rows
 * offsets[g] .. offsets[g + 1] - 1 of the flattened activations. `range` is a
 * caller-owned device buffer of G + 1 int32 holding 0, 1, ..., G, filled once
 * at initialization and reused; computing the offsets from it on the device
 * is the fix of commit df05289d (dsv4/layers/grouped_linear.py, Section A
 * detector items 2 and 5) that removes the host loop, its per-group host
 * sync and the per-call allocation. One kernel launch on `stream`.
 *   1 <= G <= 2^24, padded_rows >= 0, G * padded_rows < 2^31; 4-byte aligned
 *   pointers; ROUTER_EINVAL otherwise.
 */
int grouped_offsets(const int32_t* range, int64_t G, int64_t padded_rows, int32_t* offsets, void* stream);

/*
 * Grouped NVFP4 GEMM (the grouped linear layer of commit df05289d,
 * dsv4/layers/grouped_linear.py): for every row r of group g,
 *   out[r, n] = gsa * gsw[g] * sum_d xhat[r, d] * what_g[n, d]
 * with fp32 accumulation over exact fp16 products (the gate's arithmetic).
 *
 *   x_codes, x_scales, gsa   router_quantize outputs for the flattened
 *                            activations of all groups, [R, D] (one launch,
 *                            one global scale: the pages' fused quantize
 *                            over (G * T, D)).
 *   w_codes, w_scales, gsw   the groups' weights, [G, N, D/2], [G, N, D/16]
 *                            (each group row-major (N, K_packed), as in the
 *                            checkpoint) and [G] fp32 device scales.
 *   offsets                  [G + 1] int32 device (e.g. from
 *                            grouped_offsets): 0 = offsets[0] <= ... <=
 *                            offsets[G] <= R. Values outside are clamped
 *                            (their rows are not defined).
 *   max_rows                 host bound on any group's row count; rows of a
 *                            group past max_rows are not computed. For the
 *                            padded layout it is padded_rows.
 *   out                      [R, N] fp32; rows of no group are not written.
 * Code pointers 16-byte, scale pointers 2-byte, the rest 4-byte aligned.
 * ROUTER_EINVAL for bad sizes or pointers; ROUTER_EUNSUPPORTED for D % 32 !=
 * 0, D > ROUTER_MAX_GATE_D or a grid beyond 2^31 workgroups. One launch on
 * `stream`, no workspace, no host sync: capturable. Decode-size groups
 * (max_rows <= 4, max_rows * D <= 32768, D <= 16384) run as a stream of the
 * weights with fp16 dot products on the VALU; larger groups on fp16 MFMA
 * tiles. Both give exact products and fp32 sums in a fixed order.
 */
int grouped_gemm(const uint8_t* x_codes, const uint8_t* x_scales, const float* gsa, const uint8_t* w_codes,
                 const uint8_t* w_scales, const float* gsw, const int32_t* offsets, int64_t G, int64_t R,
                 int64_t max_rows, int64_t N, int64_t D, float* out, void* stream);

/*
 * Measurement aid, not part of the router path: reads `bytes` of `buf`
 * (device, 16-byte aligned, bytes % 16 == 0) once with 16-byte loads in one
 * launch of min(bytes / 4096 rounded up, sink_words, 8192) workgroups of 256
 * threads, and stores one XOR of the data per workgroup into `sink` (device,
 * sink_words >= 1 words). Its duration is the time a kernel needs just to
 * read that footprint, against which the gate kernels' rates are read
 * (HBM bandwidth at a gigabyte; launch and cache latency at the decode
 * gate's megabyte). Returns ROUTER_EINVAL for bad arguments.
 */
int router_probe_read(const void* buf, size_t bytes, uint32_t* sink, size_t sink_words, void* stream);

/*
 * Measurement aid, not part of the router path: 1024 workgroups of 256
 * threads (four wavefronts per SIMD on 256 compute units) each run `iters`
 * rounds of four independent 32x32x16 fp16 MFMA chains with no memory
 * traffic, then store one float per thread into `sink` (device, at least
 * 262144 floats). Its duration gives the fp16 MFMA rate the chip sustains at
 * its running clock: 1024 * 4 * iters * 4 * 32768 FLOP per launch. 1 <= iters
 * <= 2^24; ROUTER_EINVAL otherwise.
 */
int router_probe_mfma(int64_t iters, float* sink, size_t sink_floats, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_ROUTER_H */
