"""GPU backward (training step) against the fp64 oracle's chain rule.

bf16 workload: elementwise max|g - o| <= 2e-2 on dx, dK, dV, dW_up, dgamma,
dbeta, dW_mix; float32 workload: per-tensor relative error <= 1e-4.
Gradients and workspaces start as NaN, so every element (the zero rows of
absent ids included) must be written. Run twice, every gradient is bitwise
identical (no float atomics)."""
import numpy as np
import pytest

from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

NAMES = ("dx", "dK", "dV", "dW_up", "dgamma", "dbeta", "dW_mix")


def _grads_vs_oracle(name, ln_perturb=False):
    w = gu.workload(name, ln_perturb)
    if w.dy is None:
        from static_token_routed_id_amd import workloads as wl
        import dataclasses
        g = np.random.default_rng(77).standard_normal((w.batch, w.spec.d))
        w = dataclasses.replace(w, dy=wl.store(g, w.spec.dtype))
    res = gu.run(w, training=True, nan_fill=True)
    ref = gu.oracle_backward(w)
    for k in NAMES:
        got = gu.f64(res["grads"][k])
        if w.spec.dtype == "f32":
            e = gu.linf_rel(got, ref[k])
            print(f"{name} {k}: linf-rel {e:.3e}")
            assert e <= 1e-4, k
        else:
            e = gu.max_abs(got, ref[k])
            print(f"{name} {k}: max abs {e:.3e} (max |ref| "
                  f"{np.abs(ref[k]).max():.2f})")
            assert e <= 2e-2, k
    return w, res


def test_train_skew_bf16_backward():
    w, res = _grads_vs_oracle("train_skew_bf16")
    # untouched table rows are exactly zero (dK, dV started as NaN)
    used = np.zeros(w.rows, bool)
    for t in np.unique(w.ids):
        used[w.offsets[t]:w.offsets[t + 1]] = True
    for k in ("dK", "dV"):
        g = res["grads"][k].cpu().numpy()
        assert not g[~used].any(), k


@pytest.mark.parametrize("ln_perturb", [False, True])
def test_tiny_fp32_backward(ln_perturb):
    _grads_vs_oracle("tiny_fp32", ln_perturb)


def test_backward_deterministic():
    torch = gu.torch_cuda()
    w = gu.workload("train_skew_bf16")
    dev = gu.Dev(w)
    g1 = gu.run(w, dev, training=True)["grads"]
    g2 = gu.run(w, dev, training=True)["grads"]
    for k in NAMES:
        assert torch.equal(g1[k], g2[k]), k


def test_backward_deterministic_prefill_shapes():
    """Bitwise-equal reruns where the training step takes its MFMA paths
    (1024 tokens of the prefill batch, d = 1024): split-K shares added in
    order, chunk statistics combined in chunk order, one writer per dK, dV
    and dx element."""
    import dataclasses
    from static_token_routed_id_amd import workloads as wl
    torch = gu.torch_cuda()
    base = gu.workload("prefill_bf16")
    w = wl.with_ids(base, base.ids[:1024])
    g = np.random.default_rng(9).standard_normal((1024, base.spec.d))
    w = dataclasses.replace(w, dy=wl.store(g, "bf16"))
    dev = gu.Dev(w)
    g1 = gu.run(w, dev, training=True)["grads"]
    g2 = gu.run(w, dev, training=True)["grads"]
    for k in NAMES:
        assert torch.equal(g1[k], g2[k]), k


def test_backward_without_save_is_an_error():
    L = gu.lib()
    w = gu.workload("train_skew_bf16")
    dev = gu.Dev(w)
    from static_token_routed_id_amd.layer import L3Layer
    layer = L3Layer(gu.desc_of(w), w.batch, training=True)
    layer.make_plan(dev.ids, dev.offsets)
    layer.forward(*dev.params(), save=0)   # inference forward: nothing saved
    with pytest.raises(L.L3Error) as e:
        layer.backward(dev.dy, *dev.params())
    assert e.value.status == L.L3_ERR_STATE


@pytest.mark.timeout(900)
@pytest.mark.parametrize("tokens", [1024, 777])
def test_prefill_shapes_bf16_backward(tokens):
    """The training step at prefill shapes (d = 1024, d_e = 256, a table of
    171,462 rows, ids with up to 512 rows): the first 1024 tokens of the
    prefill id stream with a drawn upstream gradient, and a ragged 777
    (no multiple of the 16-token tiles or the 256-row LayerNorm blocks)."""
    import dataclasses
    from static_token_routed_id_amd import workloads as wl
    base = gu.workload("prefill_bf16")
    w = wl.with_ids(base, base.ids[:tokens])
    g = np.random.default_rng(5).standard_normal((tokens, base.spec.d))
    w = dataclasses.replace(w, dy=wl.store(g, "bf16"))
    res = gu.run(w, training=True, nan_fill=True)
    ref = gu.oracle_backward(w)
    for k in NAMES:
        got = gu.f64(res["grads"][k])
        e = gu.max_abs(got, ref[k])
        print(f"prefill shapes {k}: max abs {e:.3e} (max |ref| "
              f"{np.abs(ref[k]).max():.2f})")
        assert e <= 2e-2, k


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["prefill_bf16", "train_skew_prefill_bf16"])
def test_train_prefill_full_batch_sampled(name):
    """The training step as the training bench times it: a whole 8192-token
    batch at the prefill shapes (bf16 projections on split-K MFMA, the
    float32 operands as hi + lo halves, the segment backward on MFMA), the
    Zipf id stream and the skewed one (30% of the tokens on id 0, 512
    rows), against the oracle's steps on samples: dx of 48 tokens, dK / dV
    of eight ids (the four busiest, 512 rows each, and four drawn among the
    rest), and the whole-batch weight gradients dW_mix, dW_up, dgamma,
    dbeta."""
    import dataclasses
    from static_token_routed_id_amd import workloads as wl
    w = gu.workload(name)
    w = dataclasses.replace(w, dy=wl.upstream_grad(w))
    res = gu.run(w, training=True, nan_fill=True)
    for k in NAMES:
        assert bool(res["grads"][k].isfinite().all()), k
    rng = np.random.default_rng(5)
    tokens = np.sort(rng.choice(w.batch, 48, replace=False))
    present = np.unique(w.ids)
    ids = [int(t) for t in present[:4]] + \
        [int(t) for t in rng.choice(present[4:], 4, replace=False)]
    ref = gu.oracle_backward_sampled(w, tokens, ids)
    g = {k: gu.f64(res["grads"][k]) for k in NAMES}
    errs = {
        "dx": gu.max_abs(g["dx"][tokens], np.stack([ref["dx"][int(i)]
                                                    for i in tokens])),
        "dK": max(gu.max_abs(g["dK"][w.offsets[t]:w.offsets[t + 1]],
                             ref["dK"][t]) for t in ids),
        "dV": max(gu.max_abs(g["dV"][w.offsets[t]:w.offsets[t + 1]],
                             ref["dV"][t]) for t in ids),
    }
    for k in ("dW_mix", "dW_up", "dgamma", "dbeta"):
        errs[k] = gu.max_abs(g[k], ref[k])
    for k, e in errs.items():
        print(f"{name} full batch {k}: max abs {e:.3e}")
        assert e <= 2e-2, k


@pytest.mark.timeout(900)
def test_train_large_prefill_sampled():
    """The training step at the large-prefill shapes (d = 2048, d_e = 512,
    65536 tokens, a table of 1,759,242 rows: dK alone is 14.4 GB of
    float32), as `bench.py --train --workload large_prefill_bf16` times it.
    Every gradient starts as NaN and must come out finite; against the
    oracle's steps on samples: dx of 48 tokens, dK / dV of eight ids (the
    four most frequent, 512 rows each, and four drawn among the rest), and
    the whole-batch dW_mix, dW_up, dgamma, dbeta. Only the sampled rows of
    dK, dV and dx leave the GPU."""
    import dataclasses
    import time
    from static_token_routed_id_amd import workloads as wl
    torch = gu.torch_cuda()
    w = gu.workload("large_prefill_bf16")
    w = dataclasses.replace(w, dy=wl.upstream_grad(w))
    res = gu.run(w, training=True, nan_fill=True)
    g = res["grads"]
    for k in NAMES:
        assert bool(torch.isfinite(g[k]).all()), k
    rng = np.random.default_rng(5)
    tokens = np.sort(rng.choice(w.batch, 48, replace=False))
    present = np.unique(w.ids)
    ids = [int(t) for t in present[:4]] + \
        [int(t) for t in rng.choice(present[4:], 4, replace=False)]
    t0 = time.time()
    ref = gu.oracle_backward_sampled(w, tokens, ids)
    print(f"sampled reference in {time.time() - t0:.1f} s", flush=True)
    tix = torch.from_numpy(tokens).cuda()
    errs = {
        "dx": gu.max_abs(gu.f64(g["dx"][tix]),
                         np.stack([ref["dx"][int(i)] for i in tokens])),
        "dK": max(gu.max_abs(gu.f64(g["dK"][w.offsets[t]:w.offsets[t + 1]]),
                             ref["dK"][t]) for t in ids),
        "dV": max(gu.max_abs(gu.f64(g["dV"][w.offsets[t]:w.offsets[t + 1]]),
                             ref["dV"][t]) for t in ids),
    }
    for k in ("dW_mix", "dW_up", "dgamma", "dbeta"):
        errs[k] = gu.max_abs(gu.f64(g[k]), ref[k])
    # rows of ids absent from the batch are exactly zero
    absent = np.setdiff1d(np.arange(w.spec.vocab), present)[:64]
    for t in absent:
        r0, r1 = int(w.offsets[t]), int(w.offsets[t + 1])
        assert float(g["dK"][r0:r1].abs().max()) == 0.0
        assert float(g["dV"][r0:r1].abs().max()) == 0.0
    for k, e in errs.items():
        print(f"large prefill training {k}: max abs {e:.3e}")
        assert e <= 2e-2, k
