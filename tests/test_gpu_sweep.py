"""A sweep of shapes the fixed configurations do not take, each against the
fp64 oracle on every token (forward in both modes; backward on the small
ones): value widths that are not powers of two, hidden widths that keep the
large batches off the group kernel, batches on either side of the group
kernel's 2048-token threshold and of the small plan's 4096, a batch that
lands on exactly 4096, few ids carrying many tokens each, row caps of 1 to
512, fp32 and bf16. Each case prints its shape first. Tolerances are the
parity tests' (fp32: per-tensor relative 1e-4; bf16: elementwise absolute
2e-2)."""
import dataclasses

import numpy as np
import pytest

from static_token_routed_id_amd import workloads as wl
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

NAMES = ("dx", "dK", "dV", "dW_up", "dgamma", "dbeta", "dW_mix")

# name: Spec(dtype, vocab, zipf_s, budget, cap, d, d_e, batch, sigma_k,
# sigma_v, k_max); the seed streams are those of configuration 40 + index
CASES = [
    ("f32_cap7", "f32", 97, 1.3, 300, 7, 128, 64, 300, 1 / 8, 1 / 8, 7),
    ("bf16_d192_de128", "bf16", 1000, 0.9, 20000, 100, 192, 128, 777,
     1 / 16, 1 / 8, 100),
    ("f32_de192", "f32", 2000, 1.0, 10000, 64, 256, 192, 1500, 1 / 16,
     1 / 8, 64),
    ("bf16_group_2049", "bf16", 5000, 1.0, 1 << 17, 512, 512, 128, 2049,
     1 / 32, 1 / 16, 512),
    ("bf16_group_4096_small_plan", "bf16", 6000, 1.0, 1 << 17, 512, 512, 128,
     4096, 1 / 32, 1 / 16, 512),
    ("bf16_group_4097_radix", "bf16", 3000, 1.2, 1 << 16, 256, 1024, 256,
     4097, 1 / 32, 1 / 16, 256),
    ("bf16_few_ids_many_tokens", "bf16", 50, 0.8, 5000, 512, 512, 512, 2500,
     1 / 32, 1 / 16, 512),
    ("bf16_d768_no_group", "bf16", 40000, 1.05, 1 << 17, 512, 768, 256, 3000,
     1 / 32, 1 / 16, 512),
    ("bf16_de1024_wave", "bf16", 8000, 1.0, 1 << 16, 512, 1024, 1024, 2100,
     1 / 32, 1 / 32, 512),
    ("bf16_8193_two_passes", "bf16", 20000, 1.0, 1 << 17, 512, 512, 256,
     8193, 1 / 32, 1 / 16, 512),
    ("f32_one_token", "f32", 300, 1.0, 3000, 32, 64, 64, 1, 1 / 8, 1 / 8, 32),
    # decode-sized batches at other hidden widths: the one-wavefront plan,
    # the few-rows GEMMs, W_up's K shares summed by the LayerNorm row pass
    # (one and four 256-column chunks a wave) and the one-burst combine
    ("bf16_d1024_decode_40", "bf16", 4000, 1.0, 1 << 15, 256, 1024, 256, 40,
     1 / 32, 1 / 16, 256),
    ("bf16_d4096_decode_17", "bf16", 500, 1.0, 1 << 12, 64, 4096, 512, 17,
     1 / 64, 1 / 16, 64),
]
# small enough for the oracle's full backward
BACKWARD = ("f32_cap7", "bf16_d192_de128", "f32_de192", "f32_one_token")


def _workload(i, training=False):
    name, dt, V, s, budget, cap, d, de, B, sk, sv, kmax = CASES[i]
    spec = wl.Spec(name, dt, V, s, budget, cap, d, de, B, sk, sv,
                   training=training, k_max=kmax)
    w = wl.make_from_spec(spec, 40 + i)
    print(f"case {name}: {dt} V={V} s={s} budget={budget} cap={cap} d={d} "
          f"d_e={de} B={B} k_max={kmax} rows={w.rows}", flush=True)
    return w


@pytest.mark.parametrize("training", [False, True])
@pytest.mark.parametrize("i", range(len(CASES)),
                         ids=[c[0] for c in CASES])
def test_sweep_forward(i, training):
    w = _workload(i)
    res = gu.run(w, training=training, nan_fill=True)
    gu.check_forward(w, res, gu.oracle_forward_parallel(w, threads=8))


@pytest.mark.parametrize("name", BACKWARD)
def test_sweep_backward(name):
    i = [c[0] for c in CASES].index(name)
    w = _workload(i, training=True)
    g = np.random.default_rng(77 + i).standard_normal((w.batch, w.spec.d))
    w = dataclasses.replace(w, dy=wl.store(g, w.spec.dtype))
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
