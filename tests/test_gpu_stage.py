"""Tables in host memory: l3_stage_rows copies the batch's rows into compact
device tables and points the plan at them. The staged forward must equal
the forward over the full device tables bit for bit (same arithmetic on the
same values, only the row addresses differ); the error paths are checked
from the host (capacity too small, staging twice, backward on a staged
plan)."""
import numpy as np
import pytest

from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _host_copy(a: np.ndarray, pin=True):
    """Host tensor of a stored table (bf16 bit patterns viewed as bf16)."""
    torch = gu.torch_cuda()
    bf16 = a.dtype == np.uint16
    t = torch.from_numpy(np.ascontiguousarray(a.view(np.int16) if bf16 else a))
    if pin:
        t = t.pin_memory()
    return t.view(torch.bfloat16) if bf16 else t


def _stage_forward(w, dev, stage_rows, K_host, V_host, dma=False):
    torch = gu.torch_cuda()
    L = gu.lib()
    desc = gu.desc_of(w)
    p, _, c = L.l3_workspace_size(desc, w.batch)
    pws = torch.empty(max(p, 256), dtype=torch.uint8, device="cuda")
    scr = torch.empty(max(c, 256), dtype=torch.uint8, device="cuda")
    plan = L.l3_plan(desc, dev.ids, dev.offsets, pws)
    K_stage = torch.empty((stage_rows, w.spec.d), dtype=dev.K.dtype,
                          device="cuda")
    V_stage = torch.empty((stage_rows, w.spec.d_e), dtype=dev.V.dtype,
                          device="cuda")
    L.l3_stage_rows(plan, K_host, V_host, K_stage, V_stage, dma=dma)
    y = torch.full((w.batch, w.spec.d), float("nan"), dtype=torch.float32,
                   device="cuda")
    L.l3_forward(plan, dev.x, K_stage, V_stage, dev.W_up, dev.gamma,
                 dev.beta, dev.W_mix, y, None, scr)
    torch.cuda.synchronize()
    return plan, y, (pws, scr, K_stage, V_stage)


@pytest.mark.parametrize("dma", [False, True])
@pytest.mark.parametrize("name", ["decode_bf16", "prefill_bf16", "tiny_fp32"])
def test_staged_forward_equals_device_tables(name, dma):
    """The staged forward equals the device-table forward bit for bit, and
    both meet the oracle's bound (every token; the bf16 aggregate too)."""
    torch = gu.torch_cuda()
    L = gu.lib()
    w = gu.workload(name)
    dev = gu.Dev(w)
    ref = gu.run(w, dev)["y"]
    K_host, V_host = _host_copy(w.K), _host_copy(w.V)
    u = np.unique(w.ids)
    rows = int((w.offsets[u + 1] - w.offsets[u]).sum())
    plan, y, keep = _stage_forward(w, dev, rows, K_host, V_host, dma)
    assert L.l3_plan_check(plan) == L.L3_OK
    assert torch.equal(y, ref)
    scr = keep[1]
    res = dict(y=y, a_act=gu.aggregate_from_scratch(w, scr).clone())
    gu.check_forward(w, res, gu.oracle_forward(w))


def test_stage_errors():
    torch = gu.torch_cuda()
    L = gu.lib()
    w = gu.workload("decode_bf16")
    dev = gu.Dev(w)
    K_host, V_host = _host_copy(w.K), _host_copy(w.V)
    # capacity below the batch's rows: nothing copied, forward a no-op
    plan, y, keep = _stage_forward(w, dev, 16, K_host, V_host)
    assert L.l3_plan_check(plan) == L.L3_ERR_WORKSPACE
    assert torch.isnan(y).all()
    # a staged plan: no second staging, no backward
    u = np.unique(w.ids)
    rows = int((w.offsets[u + 1] - w.offsets[u]).sum())
    plan, y, keep = _stage_forward(w, dev, rows, K_host, V_host)
    pws, scr, K_stage, V_stage = keep
    with pytest.raises(L.L3Error) as e:
        L.l3_stage_rows(plan, K_host, V_host, K_stage, V_stage)
    assert e.value.status == L.L3_ERR_STATE
    f32 = dict(dtype=torch.float32, device="cuda")
    d, d_e = w.spec.d, w.spec.d_e
    save = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    # straight through the C ABI: the library itself refuses a backward on
    # a staged plan before it reads any buffer (the small gradient tensors
    # here would not pass the binding's shape checks)
    bufs = [dev.x, dev.x, K_stage, V_stage, dev.W_up, dev.gamma, dev.beta,
            dev.W_mix, save]
    outs = [torch.empty((w.batch, d), **f32), torch.empty((rows, d), **f32),
            torch.empty((rows, d_e), **f32), torch.empty((d, d_e), **f32),
            torch.empty(d, **f32), torch.empty(d, **f32),
            torch.empty((d, 2 * d), **f32)]
    P = lambda t: t.data_ptr()
    st = L.lib().l3_backward(plan.handle, *[P(t) for t in bufs[:-1]],
                             P(save), save.numel(), *[P(t) for t in outs],
                             P(scr), scr.numel(),
                             torch.cuda.current_stream().cuda_stream)
    assert st in (L.L3_ERR_STATE, L.L3_ERR_WORKSPACE)
    # pageable host memory is refused before any kernel runs
    L.l3_replan(plan, dev.ids, dev.offsets)
    pageable = _host_copy(w.K, pin=False)
    with pytest.raises(L.L3Error) as e:
        L.l3_stage_rows(plan, pageable, V_host, K_stage, V_stage)
    assert e.value.status == L.L3_ERR_NULL
    # a replan clears the staging: the same handle stages again
    L.l3_replan(plan, dev.ids, dev.offsets)
    L.l3_stage_rows(plan, K_host, V_host, K_stage, V_stage)
    y2 = torch.empty_like(y)
    L.l3_forward(plan, dev.x, K_stage, V_stage, dev.W_up, dev.gamma,
                 dev.beta, dev.W_mix, y2, None, scr)
    torch.cuda.synchronize()
    assert L.l3_plan_check(plan) == L.L3_OK
    assert torch.equal(y2, y)


def test_stage_dma_capacity_error():
    """The DMA path knows the row count on the host: too small a staging
    table is refused before anything is queued."""
    torch = gu.torch_cuda()
    L = gu.lib()
    w = gu.workload("decode_bf16")
    dev = gu.Dev(w)
    K_host, V_host = _host_copy(w.K), _host_copy(w.V)
    with pytest.raises(L.L3Error) as e:
        _stage_forward(w, dev, 16, K_host, V_host, dma=True)
    assert e.value.status == L.L3_ERR_WORKSPACE
