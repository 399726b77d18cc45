"""Plan + forward captured into a HIP graph (through torch.cuda.CUDAGraph):
the path makes no host synchronisation, allocation or memset on the stream,
so a captured step replays to the same bits as the eager step. Each replay
writes into a NaN-filled output and is followed by an eager step, as the
graph-replay hazards call for; both mode paths of the library are covered
(the group kernel at 8192 tokens of the prefill shape, wave items and the
row-chunk combine at the decode shape)."""
import pytest
import torch

from static_token_routed_id_amd import _lib as L
from static_token_routed_id_amd.layer import L3Layer, to_device
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["prefill_bf16", "decode_bf16"])
def test_graph_replay_matches_eager(name):
    w = gu.workload(name)
    dtype = L.L3_BF16 if w.spec.dtype == "bf16" else L.L3_F32
    desc = L.make_desc(w.spec.vocab, w.rows, w.spec.d, w.spec.d_e,
                       w.spec.k_max, dtype, L.L3_F32)
    params = [to_device(getattr(w, k)) for k in
              ("x", "K", "V", "W_up", "gamma", "beta", "W_mix")]
    ids = torch.from_numpy(w.ids).cuda()
    offsets = torch.from_numpy(w.offsets).cuda()
    layer = L3Layer(desc, w.batch, training=False)
    y = torch.empty((w.batch, w.spec.d), dtype=torch.float32, device="cuda")

    def step():
        layer.make_plan(ids, offsets)
        layer.forward(*params, y=y)

    step()
    assert L.l3_plan_check(layer.plan) == L.L3_OK
    torch.cuda.synchronize()
    ref = y.clone()
    assert torch.isfinite(ref).all()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for r in range(3):
        y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref), f"replay {r}"
        step()
        torch.cuda.synchronize()
        assert torch.equal(y, ref), f"eager step after replay {r}"
