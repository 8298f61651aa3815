"""Thin ctypes binding of libnvfp4_router.so (argument marshalling only).

Every step of the path runs in the library's HIP kernels; this module only
checks tensor properties, passes device pointers and the current HIP stream,
and raises on a non-zero status. PyTorch provides the device memory and the
stream. There is no fallback: if the library is missing, every call raises.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnvfp4_router.so")

ROUTER_OK = 0
EXPORTS = ("router_workspace_bytes", "router_workspace_init", "router_quantize", "router_gate_topk",
           "router_forward", "router_forward_noalloc", "router_status_string", "router_probe_read",
           "router_probe_mfma", "lmhead_workspace_bytes", "lmhead_argmax", "grouped_offsets", "grouped_gemm")
ROUTER_ESCRATCH = -4
STATIC_SCRATCH_BYTES = 16 << 20

_lib = None


class RouterError(RuntimeError):
    pass


def load_library(path=LIB_PATH):
    """Load the shared library once and declare its C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RouterError(f"{path} is not built: run __graft_entry__.build() (hipcc, gfx950)")
    L = ctypes.CDLL(path)
    vp, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    L.router_workspace_bytes.argtypes = [i64, i64, i64, i64]
    L.router_workspace_bytes.restype = sz
    L.router_workspace_init.argtypes = [vp, sz, vp]
    L.router_workspace_init.restype = ctypes.c_int
    L.router_quantize.argtypes = [vp, i64, i64, vp, vp, vp, vp, vp, sz, vp]
    L.router_quantize.restype = ctypes.c_int
    L.router_gate_topk.argtypes = [vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, i64, i64, i64, i64, vp, vp, vp,
                                   vp, sz, vp]
    L.router_gate_topk.restype = ctypes.c_int
    L.router_forward.argtypes = [vp, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, i64, i64, vp, vp,
                                 vp, vp, sz, vp]
    L.router_forward.restype = ctypes.c_int
    L.router_forward_noalloc.argtypes = [vp, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, i64, i64, vp,
                                         vp, vp, vp]
    L.router_forward_noalloc.restype = ctypes.c_int
    L.router_status_string.argtypes = [ctypes.c_int]
    L.router_status_string.restype = ctypes.c_char_p
    L.router_probe_read.argtypes = [vp, sz, vp, sz, vp]
    L.router_probe_read.restype = ctypes.c_int
    L.router_probe_mfma.argtypes = [i64, vp, sz, vp]
    L.router_probe_mfma.restype = ctypes.c_int
    L.lmhead_workspace_bytes.argtypes = [i64, i64, i64]
    L.lmhead_workspace_bytes.restype = sz
    L.lmhead_argmax.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, vp, vp, vp, vp, sz, vp]
    L.lmhead_argmax.restype = ctypes.c_int
    L.grouped_offsets.argtypes = [vp, i64, i64, vp, vp]
    L.grouped_offsets.restype = ctypes.c_int
    L.grouped_gemm.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, vp, vp]
    L.grouped_gemm.restype = ctypes.c_int
    _lib = L
    return L


def _check(status):
    if status != ROUTER_OK:
        msg = load_library().router_status_string(status).decode()
        raise RouterError(f"status {status}: {msg}")


def _ptr(t):
    return None if t is None or t.numel() == 0 else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _device_tensor(t, name, dtypes, ndim=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise RouterError(f"{name} must be a GPU tensor")
    if t.dtype not in dtypes:
        raise RouterError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise RouterError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise RouterError(f"{name} must have {ndim} dimensions")
    return t


def workspace_bytes(T, D, E, k):
    n = load_library().router_workspace_bytes(T, D, E, k)
    if n == 0:
        raise RouterError(f"invalid sizes T={T} D={D} E={E} k={k}")
    return int(n)


class Workspace:
    """Caller-owned scratch memory; zero-filled once (its counters must start at zero)."""

    def __init__(self, nbytes, device="cuda"):
        nbytes = (int(nbytes) + 255) // 256 * 256
        self.buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
        _check(load_library().router_workspace_init(_ptr(self.buf), nbytes, _stream()))

    @classmethod
    def for_shapes(cls, shapes, device="cuda"):
        """A workspace large enough for every (T, D, E, k) in ``shapes``."""
        return cls(max(workspace_bytes(*s) for s in shapes), device)

    @property
    def nbytes(self):
        return self.buf.numel()


class NVFP4Tensor:
    """Codes [rows, D/2] uint8, scales [rows, D/16] uint8 and the global scale [1] fp32 on the GPU."""

    def __init__(self, codes, scales, gscale):
        self.codes, self.scales, self.gscale = codes, scales, gscale

    @property
    def rows(self):
        return self.codes.shape[0]

    @property
    def D(self):
        return self.codes.shape[1] * 2


def empty_nvfp4(rows, D, device="cuda"):
    return NVFP4Tensor(torch.empty((rows, D // 2), dtype=torch.uint8, device=device),
                       torch.empty((rows, D // 16), dtype=torch.uint8, device=device),
                       torch.empty(1, dtype=torch.float32, device=device))


def quantize(x, workspace, gsa_override=None, out=None):
    """router_quantize: bf16 x [rows, D] (bfloat16, or int16/uint16 bit patterns) -> NVFP4Tensor."""
    _device_tensor(x, "x", (torch.bfloat16, torch.int16, torch.uint16), ndim=2)
    rows, D = x.shape
    if out is None:
        out = empty_nvfp4(rows, D, x.device)
    if gsa_override is not None:
        _device_tensor(gsa_override, "gsa_override", (torch.float32,))
    _check(load_library().router_quantize(_ptr(x), rows, D, _ptr(gsa_override), _ptr(out.codes),
                                          _ptr(out.scales), _ptr(out.gscale), _ptr(workspace.buf),
                                          workspace.nbytes, _stream()))
    return out


def gate_topk(xq, wq, bias, k, routed_scale, workspace, want_logits=False, out=None):
    """router_gate_topk: returns (topk_idx [T,k] int32, topk_w [T,k] fp32, logits [T,E] fp32 or None)."""
    T, D = xq.rows, xq.D
    E = wq.rows
    _device_tensor(bias, "bias", (torch.float32,), ndim=1)
    for name, t in (("x codes", xq.codes), ("x scales", xq.scales), ("w codes", wq.codes),
                    ("w scales", wq.scales)):
        _device_tensor(t, name, (torch.uint8,), ndim=2)
    if wq.D != D or bias.numel() != E:
        raise RouterError("gate weights / bias do not match x")
    if out is None:
        dev = xq.codes.device
        out = (torch.empty((T, k), dtype=torch.int32, device=dev), torch.empty((T, k), dtype=torch.float32, device=dev),
               torch.empty((T, E), dtype=torch.float32, device=dev) if want_logits else None)
    idx, w, logits = out
    _check(load_library().router_gate_topk(_ptr(xq.codes), _ptr(xq.scales), _ptr(xq.gscale), _ptr(wq.codes),
                                           _ptr(wq.scales), _ptr(wq.gscale), _ptr(bias), float(routed_scale), T, D,
                                           E, k, _ptr(idx), _ptr(w), _ptr(logits), _ptr(workspace.buf),
                                           workspace.nbytes, _stream()))
    return idx, w, logits


def forward(x, wq, bias, k, routed_scale, workspace, gsa_override=None, want_logits=False, xq=None, out=None):
    """router_forward: quantize x and route it in one call.

    Returns ``(xq, (topk_idx, topk_w, logits or None))``; ``xq`` holds x's NVFP4 codes, scales and gsa.
    """
    _device_tensor(x, "x", (torch.bfloat16, torch.int16, torch.uint16), ndim=2)
    T, D = x.shape
    E = wq.rows
    _device_tensor(bias, "bias", (torch.float32,), ndim=1)
    if wq.D != D or bias.numel() != E:
        raise RouterError("gate weights / bias do not match x")
    if gsa_override is not None:
        _device_tensor(gsa_override, "gsa_override", (torch.float32,))
    if xq is None:
        xq = empty_nvfp4(T, D, x.device)
    if out is None:
        dev = x.device
        out = (torch.empty((T, k), dtype=torch.int32, device=dev), torch.empty((T, k), dtype=torch.float32, device=dev),
               torch.empty((T, E), dtype=torch.float32, device=dev) if want_logits else None)
    idx, w, logits = out
    _check(load_library().router_forward(_ptr(x), T, D, _ptr(gsa_override), _ptr(xq.codes), _ptr(xq.scales),
                                         _ptr(xq.gscale), _ptr(wq.codes), _ptr(wq.scales), _ptr(wq.gscale),
                                         _ptr(bias), float(routed_scale), E, k, _ptr(idx), _ptr(w), _ptr(logits),
                                         _ptr(workspace.buf), workspace.nbytes, _stream()))
    return xq, out


def forward_noalloc(x, wq, bias, k, routed_scale, gsa_override=None, want_logits=False, xq=None, out=None):
    """router_forward_noalloc: router_forward with the library's static scratch instead of a workspace.

    Same arguments and results as ``forward`` without ``workspace``; raises RouterError with status -4 when the
    call needs more than the 16 MiB static scratch."""
    _device_tensor(x, "x", (torch.bfloat16, torch.int16, torch.uint16), ndim=2)
    T, D = x.shape
    E = wq.rows
    _device_tensor(bias, "bias", (torch.float32,), ndim=1)
    if wq.D != D or bias.numel() != E:
        raise RouterError("gate weights / bias do not match x")
    if gsa_override is not None:
        _device_tensor(gsa_override, "gsa_override", (torch.float32,))
    if xq is None:
        xq = empty_nvfp4(T, D, x.device)
    if out is None:
        dev = x.device
        out = (torch.empty((T, k), dtype=torch.int32, device=dev), torch.empty((T, k), dtype=torch.float32, device=dev),
               torch.empty((T, E), dtype=torch.float32, device=dev) if want_logits else None)
    idx, w, logits = out
    _check(load_library().router_forward_noalloc(_ptr(x), T, D, _ptr(gsa_override), _ptr(xq.codes),
                                                 _ptr(xq.scales), _ptr(xq.gscale), _ptr(wq.codes), _ptr(wq.scales),
                                                 _ptr(wq.gscale), _ptr(bias), float(routed_scale), E, k, _ptr(idx),
                                                 _ptr(w), _ptr(logits), _stream()))
    return xq, out


def probe_read(buf, sink):
    """One streaming read of the whole of `buf` (a contiguous device tensor) by
    the library's probe kernel, one XOR per workgroup into `sink` (int32 device
    tensor); a measurement aid, not part of the router path."""
    if not (buf.is_cuda and sink.is_cuda and buf.is_contiguous() and sink.dtype == torch.int32):
        raise RouterError("probe_read: contiguous device buffer and int32 device sink required")
    nbytes = buf.numel() * buf.element_size()
    _check(load_library().router_probe_read(_ptr(buf), nbytes, _ptr(sink), sink.numel(), _stream()))


def lmhead_workspace_bytes(T, D, N):
    n = load_library().lmhead_workspace_bytes(T, D, N)
    if n == 0:
        raise RouterError(f"invalid lm_head sizes T={T} D={D} N={N}")
    return n


def lmhead_argmax(xq, wq, workspace, want_logits=False):
    """Greedy lm_head over NVFP4 x [T, D] and weights [N, D]: returns ``(idx [T] int32, logit [T] fp32, logits
    [T, N] fp32 or None)``."""
    T, D, N = xq.rows, xq.D, wq.rows
    if wq.D != D:
        raise RouterError("lm_head weights do not match x")
    dev = xq.codes.device
    idx = torch.empty(T, dtype=torch.int32, device=dev)
    logit = torch.empty(T, dtype=torch.float32, device=dev)
    logits = torch.empty((T, N), dtype=torch.float32, device=dev) if want_logits else None
    _check(load_library().lmhead_argmax(_ptr(xq.codes), _ptr(xq.scales), _ptr(xq.gscale), _ptr(wq.codes),
                                        _ptr(wq.scales), _ptr(wq.gscale), T, D, N, _ptr(idx), _ptr(logit),
                                        _ptr(logits), _ptr(workspace.buf), workspace.nbytes, _stream()))
    return idx, logit, logits


class GroupedWeights:
    """NVFP4 weights of G groups: codes [G, N, D/2], scales [G, N, D/16], global scales [G] (one per group)."""

    def __init__(self, codes, scales, gscale):
        self.codes, self.scales, self.gscale = codes, scales, gscale

    @property
    def G(self):
        return self.codes.shape[0]

    @property
    def N(self):
        return self.codes.shape[1]

    @property
    def D(self):
        return self.codes.shape[2] * 2


def quantize_grouped_weights(w, workspace):
    """Each group's bf16 weight [G, N, D] quantized with its own global scale (router_quantize per group, at
    load time) into one GroupedWeights."""
    _device_tensor(w, "w", (torch.bfloat16, torch.int16, torch.uint16), ndim=3)
    G, N, D = w.shape
    dev = w.device
    out = GroupedWeights(torch.empty((G, N, D // 2), dtype=torch.uint8, device=dev),
                         torch.empty((G, N, D // 16), dtype=torch.uint8, device=dev),
                         torch.empty(G, dtype=torch.float32, device=dev))
    for g in range(G):
        quantize(w[g], workspace, out=NVFP4Tensor(out.codes[g], out.scales[g], out.gscale[g:g + 1]))
    return out


def grouped_offsets(range_buf, padded_rows, out=None):
    """grouped_offsets: offsets [G + 1] int32 = range_buf * padded_rows on the device."""
    _device_tensor(range_buf, "range_buf", (torch.int32,), ndim=1)
    G = range_buf.numel() - 1
    if out is None:
        out = torch.empty(G + 1, dtype=torch.int32, device=range_buf.device)
    _check(load_library().grouped_offsets(_ptr(range_buf), G, int(padded_rows), _ptr(out), _stream()))
    return out


def grouped_gemm(xq, wg, offsets, max_rows, out=None):
    """grouped_gemm: out [R, N] fp32 with out[r] = gsa * gsw[g] * xhat[r] . what_g^T for the rows of group g."""
    R, D = xq.rows, xq.D
    for name, t in (("x codes", xq.codes), ("x scales", xq.scales)):
        _device_tensor(t, name, (torch.uint8,), ndim=2)
    for name, t in (("w codes", wg.codes), ("w scales", wg.scales)):
        _device_tensor(t, name, (torch.uint8,), ndim=3)
    _device_tensor(wg.gscale, "w scales", (torch.float32,), ndim=1)
    _device_tensor(offsets, "offsets", (torch.int32,), ndim=1)
    if wg.D != D or offsets.numel() != wg.G + 1:
        raise RouterError("grouped weights / offsets do not match x")
    if out is None:
        out = torch.empty((R, wg.N), dtype=torch.float32, device=xq.codes.device)
    _check(load_library().grouped_gemm(_ptr(xq.codes), _ptr(xq.scales), _ptr(xq.gscale), _ptr(wg.codes),
                                       _ptr(wg.scales), _ptr(wg.gscale), _ptr(offsets), wg.G, R, int(max_rows),
                                       wg.N, D, _ptr(out), _stream()))
    return out


MFMA_PROBE_SINK = 1024 * 256


def probe_mfma(iters, sink):
    """Back-to-back fp16 MFMAs on every SIMD (a measurement aid): 1024 * 4 * iters * 4 * 32768 FLOP."""
    if not (sink.is_cuda and sink.dtype == torch.float32 and sink.numel() >= MFMA_PROBE_SINK):
        raise RouterError("probe_mfma: fp32 device sink of at least 262144 floats required")
    _check(load_library().router_probe_mfma(int(iters), _ptr(sink), sink.numel(), _stream()))
