"""Edge cases of the layer and of the library's size limits, forward in both
modes (and backward where noted) against the fp64 oracle:

  * every id owning a single row (k_max = 1): p = 1, a = that V row, and the
    key rows get no gradient;
  * every token on one id with 512 rows (the cap), 4096 tokens at d = 512:
    the busy-id items of the group kernel take the whole batch, and the
    backward's 64-token dX_att path takes every token;
  * the widest hidden size the library takes (d = 4096) beside the
    narrowest value width (d_e = 64), bf16 and float32;
  * a value width above the group kernel's (d_e = 1024);
  * the smallest shapes the group kernel takes (d = 512, d_e = 128) on a
    batch large enough to use it;
  * batches of one and two tokens at the decode shapes.
Tolerances are the parity tests' (float32: per-tensor relative 1e-4; bf16:
elementwise absolute 2e-2)."""
import dataclasses

import numpy as np
import pytest

from static_token_routed_id_amd import workloads as wl
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

NAMES = ("dx", "dK", "dV", "dW_up", "dgamma", "dbeta", "dW_mix")

# name: (spec, config number of the seed streams)
EDGE = {
    "one_row_f32": (wl.Spec("one_row_f32", "f32", 512, 1.0, 512, 1, 64, 64,
                            1024, 1 / 8, 1 / 8, k_max=1), 20),
    "one_row_bf16": (wl.Spec("one_row_bf16", "bf16", 512, 1.0, 512, 1, 128,
                             64, 1024, 1 / 8, 1 / 8, k_max=1), 21),
    "d4096_bf16": (wl.Spec("d4096_bf16", "bf16", 64, 1.0, 512, 16, 4096, 64,
                           256, 1 / 64, 1 / 8), 22),
    "d4096_f32": (wl.Spec("d4096_f32", "f32", 64, 1.0, 512, 16, 4096, 64, 128,
                          1 / 64, 1 / 8), 23),
    "de1024_bf16": (wl.Spec("de1024_bf16", "bf16", 256, 1.0, 4096, 64, 512,
                            1024, 512, 1 / 16, 1 / 32), 24),
    "group_min_bf16": (wl.Spec("group_min_bf16", "bf16", 2048, 1.0, 1 << 15,
                               512, 512, 128, 4096, 1 / 16, 1 / 8), 25),
    "hot512_bf16": (wl.Spec("hot512_bf16", "bf16", 256, 1.1, 1 << 14, 512,
                            512, 128, 4096, 1 / 16, 1 / 8), 26),
}


def _edge(name):
    spec, cfg = EDGE[name]
    w = wl.make_from_spec(spec, cfg)
    if name == "hot512_bf16":
        assert w.offsets[1] - w.offsets[0] == 512
        w = wl.with_ids(w, np.zeros(spec.batch, np.int32))
    if name.startswith("one_row"):
        assert (np.diff(w.offsets) == 1).all()
    return w


def _with_dy(w, seed=31):
    g = np.random.default_rng(seed).standard_normal((w.batch, w.spec.d))
    return dataclasses.replace(w, dy=wl.store(g, w.spec.dtype))


@pytest.mark.parametrize("training", [False, True])
@pytest.mark.parametrize("name", sorted(EDGE))
def test_edge_forward(name, training):
    w = _edge(name)
    res = gu.run(w, training=training, nan_fill=True)
    gu.check_forward(w, res, gu.oracle_forward_parallel(w, threads=8))


@pytest.mark.parametrize("name", ["one_row_f32", "one_row_bf16",
                                  "hot512_bf16", "d4096_bf16", "d4096_f32"])
def test_edge_backward(name):
    w = _with_dy(_edge(name))
    res = gu.run(w, training=True, nan_fill=True)
    ref = gu.oracle_backward(w)
    for k in NAMES:
        got = gu.f64(res["grads"][k])
        if w.spec.dtype == "f32":
            e = gu.linf_rel(got, ref[k])
            print(f"{name} {k}: linf-rel {e:.3e}")
            assert e <= gu.F32_REL, k
        else:
            e = gu.max_abs(got, ref[k])
            print(f"{name} {k}: max abs {e:.3e}")
            assert e <= gu.BF16_ABS, k
    if name.startswith("one_row"):
        # a single row takes the whole softmax weight whatever its score:
        # no key gradient at all
        assert float(res["grads"]["dK"].abs().max()) == 0.0


@pytest.mark.parametrize("B", [1, 2])
@pytest.mark.parametrize("training", [False, True])
def test_decode_tiny_batches(B, training):
    """One token; two tokens of the same id (decode shapes)."""
    base = gu.workload("decode_bf16")
    ids = np.full(B, base.ids[0], np.int32)
    w = wl.with_ids(base, ids)
    res = gu.run(w, training=training, nan_fill=True)
    gu.check_forward(w, res, gu.oracle_forward(w))
