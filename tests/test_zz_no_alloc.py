"""router_forward_noalloc (the library's static scratch) against router_forward (a caller workspace).

Three calls in a row on one device, each smaller than the one before: the 8192-token prefill (its experts split
over workgroups, so 8 MiB of the static scratch carries logits between them), the 64-token batched decode and the
one-token decode. Every output must equal router_forward's bit for bit: the two entry points run the same kernels
on the same inputs. The one-token call is also checked against the oracle.
"""

import numpy as np
import pytest
import torch

from nvfp4_block_scaled_06_amd import router as rt
from nvfp4_block_scaled_06_amd import workloads as wl
from oracle import check, router_ref

pytestmark = pytest.mark.gpu


def log(msg):
    print(f"[no-alloc] {msg}", flush=True)


def to_dev(bits, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev)


def run_pair(cfg, dev, ws):
    c = wl.CONFIGS[cfg]
    x, w, bias = wl.make_x(cfg), wl.make_w(cfg), wl.make_bias(cfg)
    xd, bd = to_dev(x, dev), torch.from_numpy(bias).to(dev)
    wq = rt.quantize(to_dev(w, dev), ws)
    log(f"cfg {cfg}: T={c.T} D={c.D} E={c.E} k={c.k}, router_forward_noalloc then router_forward")
    a_xq, (a_idx, a_w, a_lg) = rt.forward_noalloc(xd, wq, bd, c.k, c.routed_scale, want_logits=True)
    b_xq, (b_idx, b_w, b_lg) = rt.forward(xd, wq, bd, c.k, c.routed_scale, ws, want_logits=True)
    n_xq, (n_idx, n_w, _) = rt.forward_noalloc(xd, wq, bd, c.k, c.routed_scale, want_logits=False)
    torch.cuda.synchronize()
    for name, a, b in (("codes", a_xq.codes, b_xq.codes), ("scales", a_xq.scales, b_xq.scales),
                       ("gsa", a_xq.gscale, b_xq.gscale), ("idx", a_idx, b_idx), ("w", a_w, b_w),
                       ("logits", a_lg, b_lg), ("idx without logits", n_idx, b_idx), ("w without logits", n_w, b_w),
                       ("codes without logits", n_xq.codes, b_xq.codes)):
        assert torch.equal(a.view(torch.uint8) if a.dtype == torch.float32 else a,
                           b.view(torch.uint8) if b.dtype == torch.float32 else b), f"cfg {cfg}: {name} differ"
    return x, w, bias, a_idx.cpu().numpy(), a_w.cpu().numpy()


def test_noalloc_matches_router_forward_on_shrinking_calls():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    rt.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ws = rt.Workspace.for_shapes([(c.T, c.D, c.E, c.k) for c in wl.CONFIGS.values() if c.cfg != 5] +
                                 [(c.E, c.D, c.E, c.k) for c in wl.CONFIGS.values()], dev)
    for cfg in (4, 3, 2):
        x, w, bias, idx, wts = run_pair(cfg, dev, ws)
    c = wl.CONFIGS[2]
    ref = router_ref.router_ref(x, w, bias, c.k, c.routed_scale)
    fails = check.check_topk(idx, wts, ref["s"], ref["b"], c.k, c.routed_scale)
    assert not fails, "\n".join(fails)


def test_noalloc_rejects_a_call_beyond_its_scratch():
    rt.load_library()
    dev = torch.device("cuda:0")
    T, D, E, k = 16384, 256, 256, 8
    assert rt.workspace_bytes(T, D, E, k) > rt.STATIC_SCRATCH_BYTES
    x = torch.zeros((T, D), dtype=torch.int16, device=dev)
    ws = rt.Workspace(rt.workspace_bytes(E, D, E, k), dev)
    wq = rt.quantize(torch.zeros((E, D), dtype=torch.int16, device=dev), ws)
    with pytest.raises(rt.RouterError, match="status -4"):
        rt.forward_noalloc(x, wq, torch.zeros(E, dtype=torch.float32, device=dev), k, 2.5)
