"""CPU checks of the C ABI: the library loads, exports every declared symbol, and its
host-side logic (status strings, workspace sizing, argument validation) behaves.
No call here reaches a kernel launch."""

import ctypes
import os
import re

import pytest

from conftest import ROOT
from nvfp4_block_scaled_06_amd import router as rt

HEADER = os.path.join(ROOT, "include", "nvfp4_router.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(rt.LIB_PATH):
        from nvfp4_block_scaled_06_amd import build

        build.build()
    return rt.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"defined"})


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(rt.EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    assert lib.router_status_string(0) == b"ok"
    for s in (-1, -2, -3, -4):
        assert lib.router_status_string(s) not in (b"ok", b"unknown status")
    assert lib.router_status_string(7) == b"unknown status"
    assert b"D % 32" in lib.router_status_string(-2)


STATE = 4096 + 128 * 1024  # counters + the decode region: zero between calls


def test_workspace_bytes(lib):
    n = lib.router_workspace_bytes(1, 7168, 256, 8)
    assert n >= STATE and n % 4 == 0
    assert lib.router_workspace_bytes(64, 7168, 256, 8) >= lib.router_workspace_bytes(1, 7168, 256, 8)
    assert lib.router_workspace_bytes(8192, 7168, 256, 8) == STATE + 8192 * 256 * 4  # split experts: [T, E] logits
    assert lib.router_workspace_bytes(32768, 7168, 384, 8) == STATE + 4096  # all experts per workgroup: quantizer only
    assert lib.router_workspace_bytes(1, 7168, 256, 8) == STATE + 4096  # decode: its region, and the quantizer's
    for bad in [(1, 7168, 256, 0), (1, 7168, 256, 257), (1, 7169, 256, 8), (-1, 7168, 256, 8), (1, 7168, 0, 1),
                (1, 7168, 513, 8)]:
        assert lib.router_workspace_bytes(*bad) == 0, bad


FAKE = ctypes.c_void_p(1 << 20)  # aligned, never dereferenced: validation fails first


def test_quantize_rejects_bad_arguments(lib):
    q = lib.router_quantize
    assert q(FAKE, 4, 24, None, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == -1  # D % 16
    assert q(FAKE, 4, 0, None, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == -1
    assert q(FAKE, -1, 256, None, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == -1
    assert q(None, 4, 256, None, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == -1
    assert q(ctypes.c_void_p((1 << 20) + 8), 4, 256, None, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == -1
    # Two-pass sizes need workspace scratch.
    assert q(FAKE, 4096, 7168, None, FAKE, FAKE, FAKE, None, 0, None) == -1
    assert q(FAKE, 4096, 7168, None, FAKE, FAKE, FAKE, FAKE, 256, None) == -1


def test_gate_rejects_bad_arguments(lib):
    g = lib.router_gate_topk
    args = dict(xc=FAKE, xs=FAKE, gsa=FAKE, wc=FAKE, ws=FAKE, gsw=FAKE, bias=FAKE, r=2.5, T=1, D=7168, E=256, k=8,
                idx=FAKE, w=FAKE, logits=None, work=FAKE, nbytes=1 << 20, stream=None)

    def call(**kw):
        a = dict(args, **kw)
        return g(*a.values())

    assert call(D=7176) == -1  # D % 16
    assert call(D=7184) == -2  # D % 32: documented as unsupported by the gate kernels
    assert call(D=(1 << 22) + 32, T=300) == -2  # beyond ROUTER_MAX_GATE_D
    assert call(k=0) == -1 and call(k=257) == -1
    assert call(E=600, k=8) == -2
    assert call(k=33, E=256) == -2
    assert call(bias=None) == -1
    assert call(xc=ctypes.c_void_p((1 << 20) + 4)) == -1
    assert call(work=None, nbytes=0) == -1  # split gate needs its counters
    assert call(nbytes=100) == -1


def test_probe_rejects_bad_arguments(lib):
    buf, sink = ctypes.c_void_p(0x10000), ctypes.c_void_p(0x20000)
    assert lib.router_probe_read(None, 4096, sink, 16, None) == -1
    assert lib.router_probe_read(buf, 4096, None, 16, None) == -1
    assert lib.router_probe_read(buf, 4096, sink, 0, None) == -1
    assert lib.router_probe_read(buf, 4100, sink, 16, None) == -1  # not a multiple of 16 bytes
    assert lib.router_probe_read(ctypes.c_void_p(0x10008), 4096, sink, 16, None) == -1  # misaligned
    assert lib.router_probe_read(buf, 0, sink, 16, None) == -1


def test_lmhead_workspace_and_validation(lib):
    # counters + one 8-byte candidate per token and 64-row workgroup
    assert lib.lmhead_workspace_bytes(1, 7168, 129280) == STATE + 8 * 2020
    assert lib.lmhead_workspace_bytes(4, 7168, 65) == STATE + 8 * 4 * 2
    for bad in [(5, 7168, 10), (1, 7160, 10), (1, 16416, 10), (1, 7168, 0), (-1, 7168, 10), (4, 16384, 10)]:
        assert lib.lmhead_workspace_bytes(*bad) == 0, bad
    p = ctypes.c_void_p(0x100000)
    args = [p, p, p, p, p, p, 1, 7168, 100, p, p, None, p, 1 << 20, None]
    bad_d = list(args); bad_d[7] = 7160
    assert lib.lmhead_argmax(*bad_d) == -1
    no_ws = list(args); no_ws[12] = None
    assert lib.lmhead_argmax(*no_ws) == -1
    small_ws = list(args); small_ws[13] = 100
    assert lib.lmhead_argmax(*small_ws) == -1
    odd = list(args); odd[0] = ctypes.c_void_p(0x100008)  # x codes not 16-byte aligned
    assert lib.lmhead_argmax(*odd) == -1
    empty = list(args); empty[6] = 0
    assert lib.lmhead_argmax(*empty) == 0  # T == 0: nothing to do


def test_mfma_probe_rejects_bad_arguments(lib):
    sink = ctypes.c_void_p(0x100000)
    assert lib.router_probe_mfma(0, sink, 1 << 20, None) == -1
    assert lib.router_probe_mfma(100, None, 1 << 20, None) == -1
    assert lib.router_probe_mfma(100, sink, 1000, None) == -1  # sink smaller than one float per thread
    assert lib.router_probe_mfma(1 << 25, sink, 1 << 20, None) == -1


def test_noalloc_rejects_sizes_beyond_its_static_scratch(lib):
    """router_forward_noalloc refuses, before touching the GPU, a call whose scratch exceeds the 16 MiB array,
    and passes invalid sizes on to router_forward's own checks."""
    T, D, E, k = 16384, 7168, 256, 8  # prefill with split experts: [T, E] fp32 logits = 16 MiB + counters
    assert lib.router_workspace_bytes(T, D, E, k) > rt.STATIC_SCRATCH_BYTES
    args = [FAKE, T, D, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2.5, E, k, FAKE, FAKE, None, None]
    assert lib.router_forward_noalloc(*args) == rt.ROUTER_ESCRATCH
    assert b"16 MiB" in lib.router_status_string(rt.ROUTER_ESCRATCH)
    bad = list(args); bad[2] = 7176  # D % 16
    assert lib.router_forward_noalloc(*bad) == -1
    bad = list(args); bad[1] = 1; bad[12] = 600  # E > 512
    assert lib.router_forward_noalloc(*bad) == -2


def test_grouped_entry_points_reject_bad_arguments(lib):
    p = ctypes.c_void_p(0x100000)
    assert lib.grouped_offsets(p, 0, 4, p, None) == -1  # G >= 1
    assert lib.grouped_offsets(p, 8, -1, p, None) == -1
    assert lib.grouped_offsets(None, 8, 4, p, None) == -1
    assert lib.grouped_offsets(p, 1 << 20, 1 << 12, p, None) == -1  # G * padded_rows >= 2^31
    args = [p, p, p, p, p, p, p, 8, 8, 1, 4096, 7168, p, None]

    def call(i, v):
        a = list(args)
        a[i] = v
        return lib.grouped_gemm(*a)

    assert call(7, 0) == -1  # G
    assert call(11, 7176) == -1  # D % 16
    assert call(11, 7184) == -2  # D % 32: the MFMA tiles read 32-element chunks
    assert call(6, None) == -1  # offsets
    assert call(0, ctypes.c_void_p(0x100008)) == -1  # x codes not 16-byte aligned
    assert call(10, 0) == -1  # N
    assert call(8, 0) == 0  # no rows: nothing to do
    assert call(9, 0) == 0  # no rows per group: nothing to do
