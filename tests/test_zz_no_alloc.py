"""pisa_forward_noalloc (the forward pass on the library's static per-GPU workspace) through the C
ABI: two calls in a row, the second on a smaller layer, each bit-identical to pisa_forward with an
attached workspace on the same inputs; a plan too large for the static workspace is refused."""

import ctypes

import pytest
import torch

from pisa_cases import log
from sparse_attention_diffusion_pool_amd import _lib as L
from workloads import custom, layer_inputs, workload

pytestmark = pytest.mark.gpu


def _both(w):
    dev = torch.device("cuda", 0)
    qd, kd, vd = (t.to(dev) for t in layer_inputs(w))
    H, Lq, d = qd.shape
    ref_plan = L.Plan(Lq, H, d, w.B, w.keep)
    ref_plan.attach_workspace(device=dev)
    ref = torch.full_like(qd, float("nan"))
    ref_plan.forward(qd, kd, vd, ref)
    plan = L.Plan(Lq, H, d, w.B, w.keep)  # no workspace attached
    out = torch.full_like(qd, float("nan"))
    log(f"[noalloc] {w.name} H={H} L={Lq} B={w.B} workspace={plan.info()['workspace_bytes']} bytes")
    plan.forward_noalloc(qd, kd, vd, out)
    torch.cuda.synchronize()
    ref_plan.destroy()
    plan.destroy()
    return out, ref


def test_noalloc_matches_forward_on_two_calls():
    big = workload("wan480p-like-L32760")
    small = custom("noalloc-small-B64", 2, (13, 10), 128, 64, 0.5, "bf16")
    for w in (big, small):
        out, ref = _both(w)
        assert torch.isfinite(out.float()).all(), w.name
        assert torch.equal(out, ref), f"{w.name}: pisa_forward_noalloc differs from pisa_forward"


def test_noalloc_refuses_plans_beyond_the_static_workspace():
    lib = L.load()
    p = L.Plan(75600, 40, 128, 128, 0.10, first_order=L.FIRST_ORDER_BLOCK)  # H_j^T of every block: ~1.6 GB
    assert p.info()["workspace_bytes"] > 96 << 20
    a = ctypes.c_void_p(1 << 20)
    assert lib.pisa_forward_noalloc(p.handle, a, a, a, a, None) == 4
    assert "static workspace" in L.last_error()
    p.destroy()
