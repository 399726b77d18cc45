"""L3Function, the torch.autograd wrapper, against the fp64 oracle: y from
the forward, and every input's gradient after (y * dy).sum().backward().

float32 workload: per-tensor relative error <= 1e-4. bf16 workload: the
gradients come back in the inputs' dtype (autograd's rule), so the bound is
the library's float32 bound plus the rounding to bf16 of the result:
|g - o| <= 2e-2 + 2^-8 |o|. A second forward through the same layer object
before the first one's backward re-plans it, and that backward raises."""
import dataclasses

import numpy as np
import pytest

from static_token_routed_id_amd import workloads as wl
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

LEAVES = ("x", "K", "V", "W_up", "gamma", "beta", "W_mix")
GRAD = dict(x="dx", K="dK", V="dV", W_up="dW_up", gamma="dgamma",
            beta="dbeta", W_mix="dW_mix")


def _setup(name):
    torch = gu.torch_cuda()
    from static_token_routed_id_amd.layer import L3Layer
    w = gu.workload(name)
    if w.dy is None:
        w = dataclasses.replace(w, dy=wl.upstream_grad(w))
    dev = gu.Dev(w)
    leaves = {k: getattr(dev, k).clone().requires_grad_(True) for k in LEAVES}
    layer = L3Layer(gu.desc_of(w), w.batch, training=True)
    dy = dev.dy.float()
    return torch, w, dev, leaves, layer, dy


@pytest.mark.parametrize("name", ["tiny_fp32", "train_skew_bf16"])
def test_l3function_matches_oracle(name):
    torch, w, dev, leaves, layer, dy = _setup(name)
    from static_token_routed_id_amd.layer import L3Function
    y = L3Function.apply(layer, dev.ids, dev.offsets,
                         *[leaves[k] for k in LEAVES])
    (y * dy).sum().backward()
    torch.cuda.synchronize()
    gu.check_forward(w, dict(y=y.detach()), gu.oracle_forward(w))
    ref = gu.oracle_backward(w)
    for k in LEAVES:
        g = leaves[k].grad
        assert g is not None and g.dtype == leaves[k].dtype, k
        got, want = gu.f64(g), ref[GRAD[k]]
        if w.spec.dtype == "f32":
            e = gu.linf_rel(got, want)
            print(f"{name} {k}.grad: linf-rel {e:.3e}")
            assert e <= gu.F32_REL, k
        else:
            excess = np.abs(got - want) - 2 ** -8 * np.abs(want)
            e = float(excess.max())
            print(f"{name} {k}.grad: max(|g - o| - 2^-8 |o|) {e:.3e}")
            assert e <= gu.BF16_ABS, k


def test_l3function_replan_before_backward_raises():
    torch, w, dev, leaves, layer, dy = _setup("train_skew_bf16")
    from static_token_routed_id_amd.layer import L3Function
    args = [leaves[k] for k in LEAVES]
    y1 = L3Function.apply(layer, dev.ids, dev.offsets, *args)
    y2 = L3Function.apply(layer, dev.ids, dev.offsets, *args)
    with pytest.raises(RuntimeError, match="re-planned"):
        (y1 * dy).sum().backward()
    # the latest forward's backward still works
    (y2 * dy).sum().backward()
    torch.cuda.synchronize()
    assert leaves["x"].grad is not None


def test_binding_rejects_bad_arguments():
    """The binding checks dtype, device, contiguity and shape before an
    address crosses the C ABI: int64 ids, int32 offsets, a parameter of the
    wrong dtype or shape, a transposed view and a host tensor all raise."""
    torch = gu.torch_cuda()
    L = gu.lib()
    w = gu.workload("train_skew_bf16")
    dev = gu.Dev(w)
    from static_token_routed_id_amd.layer import L3Layer
    layer = L3Layer(gu.desc_of(w), w.batch, training=True)
    with pytest.raises(TypeError):
        layer.make_plan(dev.ids.long(), dev.offsets)
    with pytest.raises((TypeError, ValueError)):
        layer.make_plan(dev.ids, dev.offsets.int())
    with pytest.raises(ValueError):
        layer.make_plan(dev.ids, dev.offsets[:-1])
    with pytest.raises(ValueError):
        layer.make_plan(dev.ids.cpu(), dev.offsets)
    layer.make_plan(dev.ids, dev.offsets)
    p = list(dev.params())
    bad = [(0, p[0].float()),            # x in float32 on a bf16 layer
           (3, p[3].t()),                # W_up transposed (not contiguous)
           (6, p[6][:, :w.spec.d].contiguous()),   # W_mix of the wrong shape
           (1, p[1].cpu())]              # K in host memory
    for i, t in bad:
        q = list(p)
        q[i] = t
        with pytest.raises((TypeError, ValueError)):
            layer.forward(*q)
    y = torch.empty((w.batch, w.spec.d), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(TypeError):
        layer.forward(*p, y=y)           # y in bf16 on a float32-output desc
    layer.forward(*p)
    torch.cuda.synchronize()
    assert L.l3_plan_check(layer.plan) == L.L3_OK
