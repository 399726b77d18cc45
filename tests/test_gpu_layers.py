"""One plan shared by a stack of layers (the ids, and so the sort and the
segments, are the same for every layer of a model; each layer has its own
tables and weights over the same offsets).

* inference: the plan is made on a side stream while other work runs on the
  main stream; two layers' forwards on the main stream (after an event) are
  each checked against the oracle on sampled tokens, and are bitwise equal to
  forwards with a plan of their own;
* training: two layers' saving forwards, then both backward passes, each
  layer's gradients against the oracle (bf16: max abs <= 2e-2).
"""
import numpy as np
import pytest

from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

NAMES = ("dx", "dK", "dV", "dW_up", "dgamma", "dbeta", "dW_mix")


def _workspaces(desc, B, training):
    torch = gu.torch_cuda()
    L = gu.lib()
    p, s, c = L.l3_workspace_size(desc, B)
    u8 = dict(dtype=torch.uint8, device="cuda")
    return (torch.empty(max(p, 256), **u8),
            torch.empty(max(s, 256), **u8) if training else None,
            torch.empty(max(c, 256), **u8))


@pytest.mark.timeout(600)
def test_plan_shared_by_layers_forward():
    torch = gu.torch_cuda()
    L = gu.lib()
    from static_token_routed_id_amd import workloads as wl
    w0 = gu.workload("prefill_bf16")
    layers = [w0, wl.layer_params(w0, 1)]
    devs = [gu.Dev(w) for w in layers]
    desc = gu.desc_of(w0)
    pws, _, scr = _workspaces(desc, w0.batch, False)
    # the plan on a side stream, overlapping unrelated work on the main one
    side = torch.cuda.Stream()
    a = torch.randn(4096, 4096, device="cuda")
    done = torch.cuda.Event()
    side.wait_stream(torch.cuda.current_stream())
    busy = a @ a
    with torch.cuda.stream(side):
        plan = L.l3_plan(desc, devs[0].ids, devs[0].offsets, pws, stream=side)
        done.record(side)
    torch.cuda.current_stream().wait_event(done)
    ys = []
    for dev in devs:
        y = torch.empty((w0.batch, w0.spec.d), dtype=torch.float32,
                        device="cuda")
        L.l3_forward(plan, *dev.params(), y, None, scr)
        ys.append(y)
    torch.cuda.synchronize()
    del busy
    assert L.l3_plan_check(plan) == L.L3_OK
    rng = np.random.default_rng(3)
    tokens = np.unique(rng.choice(w0.batch, 384, replace=False))
    for i, (w, y) in enumerate(zip(layers, ys)):
        ref = gu.oracle_forward(w, tokens=tokens)
        e = gu.max_abs(gu.f64(y)[tokens], ref["y"])
        print(f"layer {i}: y max abs {e:.3e}")
        assert e <= 2e-2, i
        # the same as a plan of its own
        own = gu.run(w, devs[i])["y"]
        assert torch.equal(own, y), i


def test_plan_shared_by_layers_training():
    torch = gu.torch_cuda()
    L = gu.lib()
    from static_token_routed_id_amd import workloads as wl
    w0 = gu.workload("train_skew_bf16")
    layers = [w0, wl.layer_params(w0, 1)]
    devs = [gu.Dev(w) for w in layers]
    desc = gu.desc_of(w0)
    pws, _, scr = _workspaces(desc, w0.batch, False)
    saves = [_workspaces(desc, w0.batch, True)[1] for _ in layers]
    plan = L.l3_plan(desc, devs[0].ids, devs[0].offsets, pws)
    f32 = dict(dtype=torch.float32, device="cuda")
    B, d, d_e, R = w0.batch, w0.spec.d, w0.spec.d_e, w0.rows
    for dev, save in zip(devs, saves):
        y = torch.empty((B, d), **f32)
        L.l3_forward(plan, *dev.params(), y, save, scr)
    grads = []
    for dev, save in zip(devs, saves):
        g = dict(dx=torch.empty((B, d), **f32), dK=torch.empty((R, d), **f32),
                 dV=torch.empty((R, d_e), **f32),
                 dW_up=torch.empty((d, d_e), **f32),
                 dgamma=torch.empty(d, **f32), dbeta=torch.empty(d, **f32),
                 dW_mix=torch.empty((d, 2 * d), **f32))
        L.l3_backward(plan, devs[0].dy, *dev.params(), save, g["dx"],
                      g["dK"], g["dV"], g["dW_up"], g["dgamma"], g["dbeta"],
                      g["dW_mix"], scr)
        grads.append(g)
    torch.cuda.synchronize()
    for i, (w, g) in enumerate(zip(layers, grads)):
        ref = gu.oracle_backward(w)
        for k in NAMES:
            e = gu.max_abs(gu.f64(g[k]), ref[k])
            print(f"layer {i} {k}: max abs {e:.3e}")
            assert e <= 2e-2, (i, k)
