"""l3_forward_noalloc (the inference forward with its scratch in the
library's static device array) against l3_forward with a caller workspace:
the same kernels on the same inputs, so y must be identical bit for bit, on
two calls in a row, the second with a smaller batch (the array keeps the
first call's contents); both within the oracle's bound. A batch whose
forward needs more scratch than the array holds is refused before any
device work."""
import numpy as np
import pytest

from static_token_routed_id_amd import workloads as wl
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _plan(w, dev):
    torch = gu.torch_cuda()
    L = gu.lib()
    desc = gu.desc_of(w)
    p, _, _ = L.l3_workspace_size(desc, w.batch)
    ws = torch.empty(max(p, 256), dtype=torch.uint8, device="cuda")
    return L.l3_plan(desc, dev.ids, dev.offsets, ws), ws


@pytest.mark.parametrize("name", ["decode_bf16", "tiny_fp32"])
def test_noalloc_matches_forward_twice(name):
    torch = gu.torch_cuda()
    L = gu.lib()
    base = gu.workload(name)
    small = wl.with_ids(base, base.ids[:41])
    for w in (base, small):      # the second call has fewer tokens
        dev = gu.Dev(w)
        want = gu.run(w, dev, nan_fill=True)["y"]
        plan, keep = _plan(w, dev)
        y = torch.full_like(want, float("nan"))
        L.l3_forward_noalloc(plan, *dev.params(), y)
        torch.cuda.synchronize()
        assert L.l3_plan_check(plan) == L.L3_OK
        print(f"{name} B={w.batch}: noalloc y equal: "
              f"{bool(torch.equal(y, want))}", flush=True)
        assert torch.equal(y, want)
        gu.check_forward(w, dict(y=y), gu.oracle_forward(w))


def test_noalloc_refuses_too_large_a_batch():
    torch = gu.torch_cuda()
    L = gu.lib()
    w = gu.workload("prefill_bf16")          # 8192 tokens, d = 1024
    dev = gu.Dev(w)
    _, _, c = L.l3_workspace_size(gu.desc_of(w), w.batch)
    assert c > L.L3_NOALLOC_SCRATCH_BYTES
    plan, keep = _plan(w, dev)
    y = torch.full((w.batch, w.spec.d), float("nan"), device="cuda")
    with pytest.raises(L.L3Error) as e:
        L.l3_forward_noalloc(plan, *dev.params(), y)
    assert e.value.status == L.L3_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool(torch.isnan(y).all())
