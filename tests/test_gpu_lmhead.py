"""GPU parity of the greedy lm_head GEMV (lmhead_argmax) against the oracle.

Small shapes are compared in full (every logit within 1e-5 of the |x||w|
scale, the chosen row under the near-tie rule). At the vocabulary size
(129,280 rows x 7168) the oracle checks sampled rows, the chosen row and the
rows whose device logits come closest to it; the chosen row must also be the
first maximum of the device's own logits.
"""

import numpy as np
import pytest
import torch

from nvfp4_block_scaled_06_amd import router as rt
from nvfp4_block_scaled_06_amd import workloads as wl
from oracle import check, lmhead_ref, quant_ref, router_ref

pytestmark = pytest.mark.gpu

VOCAB = 129280  # rows of the full-size case (a DeepSeek-sized vocabulary; 1.85 GB as BF16)


def log(msg):
    print(f"[gpu-lmhead] {msg}", flush=True)


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    rt.load_library()
    d = torch.device("cuda:0")
    torch.cuda.set_device(d)
    return d


def quantize_dev(bits_dev, ws):
    q = rt.quantize(bits_dev, ws)
    torch.cuda.synchronize()
    return q


def host(q):
    return q.codes.cpu().numpy(), q.scales.cpu().numpy(), q.gscale.cpu().numpy()[0]


def workspace(dev, T, D, N):
    return rt.Workspace(max(rt.lmhead_workspace_bytes(T, D, N), rt.workspace_bytes(N, D, 1, 1),
                            rt.workspace_bytes(T, D, 1, 1)), dev)


def synth_bits(shape, seed, scale):
    a = np.random.default_rng(seed).standard_normal(shape, dtype=np.float32) * np.float32(scale)
    return wl.bf16_bits(a)


def to_dev(bits, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev)


def run_full_check(dev, x_bits, w_bits, what):
    T, D = x_bits.shape
    N = w_bits.shape[0]
    ws = workspace(dev, T, D, N)
    xq, wq = quantize_dev(to_dev(x_bits, dev), ws), quantize_dev(to_dev(w_bits, dev), ws)
    idx, logit, logits = rt.lmhead_argmax(xq, wq, ws, want_logits=True)
    torch.cuda.synchronize()
    L, A = router_ref.logits_ref(*host(xq), *host(wq))
    fails = check.check_logits(logits.cpu().numpy(), L, A)
    fails += lmhead_ref.check_argmax(idx.cpu().numpy(), logit.cpu().numpy(), L, A)
    assert not fails, f"{what}:\n" + "\n".join(fails[:10])
    return idx.cpu().numpy()


@pytest.mark.parametrize("T,D,N", [
    (1, 7168, 5000),   # decode, a vocabulary slice
    (4, 7168, 777),    # largest T, ragged last workgroup
    (3, 1056, 65),     # 33 chunks per row (ragged lane chunks), 2 workgroups
    (2, 32, 1),        # smallest D and N
    (1, 16384, 300),   # largest D (8 chunks per lane)
])
def test_lmhead_matches_oracle(dev, T, D, N):
    log(f"lmhead T={T} D={D} N={N}")
    run_full_check(dev, synth_bits((T, D), 11 + T, 1.0), synth_bits((N, D), 97 + N, 0.02), f"T={T} D={D} N={N}")


def test_lmhead_exact_tie_goes_to_lower_row(dev):
    T, D, N = 2, 2048, 300
    x = synth_bits((T, D), 5, 1.0)
    w = synth_bits((N, D), 6, 0.02)
    # Rows 40 and 200 are the same vector aligned with token 0: identical codes, identical logits, the maximum.
    xv = wl.bf16_to_f32(x[0])
    w[40] = w[200] = wl.bf16_bits(np.sign(xv) * np.float32(0.05))
    idx = run_full_check(dev, x, w, "tie")
    assert idx[0] == 40


def test_lmhead_full_vocabulary_sampled(dev):
    T, D, N = 1, 7168, VOCAB
    log(f"lmhead full size N={N}")
    ws = workspace(dev, T, D, N)
    g = torch.Generator(device=dev).manual_seed(1234)
    w = torch.randn((N, D), generator=g, device=dev, dtype=torch.bfloat16)
    wq = quantize_dev(w, ws)
    del w
    x_bits = synth_bits((T, D), 4321, 1.0)
    xq = quantize_dev(to_dev(x_bits, dev), ws)
    idx, logit, logits = rt.lmhead_argmax(xq, wq, ws, want_logits=True)
    torch.cuda.synchronize()
    idx, logit, Lg = int(idx.cpu()[0]), float(logit.cpu()[0]), logits.cpu().numpy()[0]
    # The device's choice is the first maximum of its own logits, and its logit is that row's.
    assert idx == int(np.argmax(Lg)) and logit == float(Lg[idx])
    # The oracle on sampled rows, the chosen row and the 32 rows closest to it.
    rows = np.unique(np.concatenate([wl.sample_rows(N, 256, seed=5), np.argsort(-Lg)[:33]]))
    wc, wsb, gsw = host(wq)
    L, A = router_ref.logits_ref(*host(xq), wc[rows], wsb[rows], gsw)
    fails = check.check_logits(Lg[rows][None, :], L, A)
    sel = np.searchsorted(rows, idx)
    fails += lmhead_ref.check_argmax(np.array([sel]), np.array([logit]), L, A)
    assert not fails, "\n".join(fails[:10])


@pytest.mark.gpu
def test_lmhead_weights_past_32bit_offsets(dev):
    """N x D/2 code bytes above 2^32 (4.3 GB, past any 32-bit byte offset from the matrix's start): the loads'
    buffer ranges and offsets are per workgroup, so rows far into the matrix read their own bytes. The oracle on
    sampled rows, the last 64 rows and the 33 rows with the largest device logits."""
    T, D, N = 1, 16384, (1 << 19) + 3
    assert N * D // 2 > (1 << 32)
    log(f"lmhead N={N} D={D}: {N * D // 2} code bytes")
    ws = workspace(dev, T, D, N)
    g = torch.Generator(device=dev).manual_seed(77)
    w = torch.randn((N, D), generator=g, device=dev, dtype=torch.bfloat16)
    wq = quantize_dev(w, ws)
    x_bits = synth_bits((T, D), 7654, 1.0)
    xq = quantize_dev(to_dev(x_bits, dev), ws)
    idx, logit, logits = rt.lmhead_argmax(xq, wq, ws, want_logits=True)
    torch.cuda.synchronize()
    idx, logit, Lg = int(idx.cpu()[0]), float(logit.cpu()[0]), logits.cpu().numpy()[0]
    assert idx == int(np.argmax(Lg)) and logit == float(Lg[idx])
    rows = np.unique(np.concatenate([wl.sample_rows(N, 128, seed=9), np.arange(N - 64, N),
                                     np.argsort(-Lg)[:33]]))
    ri = torch.from_numpy(rows).to(dev)
    # Codes of the sampled rows against the oracle's under the device's global scale, whose value is checked
    # against the tensor's max on its own.
    wc, wsb, gsw = wq.codes[ri].cpu().numpy(), wq.scales[ri].cpu().numpy(), wq.gscale.cpu().numpy()[0]
    amax = float(w.abs().max().float().cpu())
    assert gsw == quant_ref.gsa_ref(amax)
    wr = quant_ref.quantize_ref(w[ri].view(torch.int16).cpu().numpy().view(np.uint16), gsa_override=gsw)
    del w
    fails = check.check_quant(wc, wsb, gsw, wr)
    L, A = router_ref.logits_ref(*host(xq), wc, wsb, gsw)
    fails += check.check_logits(Lg[rows][None, :], L, A)
    sel = np.searchsorted(rows, idx)
    fails += lmhead_ref.check_argmax(np.array([sel]), np.array([logit]), L, A)
    assert not fails, "\n".join(fails[:10])

