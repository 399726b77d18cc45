"""GPU forward against the fp64 oracle on the same (rounded) inputs.

Tolerances: float32 workloads -- per-tensor relative error
max|g - o| / max|o| <= 1e-4; bf16 workloads -- elementwise max|g - o| <= 2e-2
on y (float32 output). The aggregate a = V_t^T Softmax(K_t x) is also
checked directly (saved float32 copy), so LayerNorm and W_mix cannot hide
an aggregation error."""
import numpy as np
import pytest

from static_token_routed_id_amd import workloads as wl
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

F32_REL = 1e-4
BF16_ABS = 2e-2
A_BF16_ABS = 2e-3   # the aggregate itself (|a| < 0.3 on these inputs)


def _check(w, res, ref, tokens=None):
    y = gu.f64(res["y"])
    a = gu.f64(res["a32"]) if "a32" in res else None
    if tokens is not None:
        y = y[tokens]
        a = a[tokens] if a is not None else None
    if w.spec.dtype == "f32":
        ey = gu.linf_rel(y, ref["y"])
        print(f"{w.spec.name}: y linf-rel {ey:.3e}")
        assert ey <= F32_REL
        if a is not None:
            ea = gu.linf_rel(a, ref["a"])
            print(f"{w.spec.name}: a linf-rel {ea:.3e}")
            assert ea <= F32_REL
    else:
        ey = gu.max_abs(y, ref["y"])
        print(f"{w.spec.name}: y max abs {ey:.3e} (max|y| "
              f"{np.abs(ref['y']).max():.2f})")
        assert ey <= BF16_ABS
        if a is not None:
            ea = gu.max_abs(a, ref["a"])
            print(f"{w.spec.name}: a max abs {ea:.3e}")
            assert ea <= A_BF16_ABS


@pytest.mark.parametrize("ln_perturb", [False, True])
def test_tiny_fp32(ln_perturb):
    w = gu.workload("tiny_fp32", ln_perturb)
    res = gu.run(w, training=True)
    _check(w, res, gu.oracle_forward(w))


@pytest.mark.parametrize("training", [False, True])
def test_prefill_bf16(training):
    """Inference (bf16 u; LayerNorm folded into W_mix from per-tile row
    statistics of the W_up epilogue) and training (float32 u, saved state)
    paths."""
    w = gu.workload("prefill_bf16", True)
    res = gu.run(w, training=training)
    _check(w, res, gu.oracle_forward(w))


def test_prefill_bf16_ragged_small_and_large_plan():
    base = gu.workload("prefill_bf16")
    for B in (1000, 8193):
        ids = wl.batch_ids(base.spec, 1, B + 7)[7:]
        w = wl.with_ids(base, ids)
        print(f"ragged B={B}", flush=True)
        res = gu.run(w, training=True)
        _check(w, res, gu.oracle_forward(w))


def test_prefill_bf16_output_bf16():
    """bf16 y is the float32 y rounded to nearest even, bit for bit."""
    torch = gu.torch_cuda()
    L = gu.lib()
    w = gu.workload("prefill_bf16", True)
    dev = gu.Dev(w)
    y32 = gu.run(w, dev)["y"]
    y16 = gu.run(w, dev, y_dtype=L.L3_BF16)["y"]
    assert y16.dtype == torch.bfloat16
    assert torch.equal(y16, y32.to(torch.bfloat16))


def test_decode_bf16():
    w = gu.workload("decode_bf16")
    res = gu.run(w, training=True)
    _check(w, res, gu.oracle_forward(w))


@pytest.mark.timeout(900)
def test_large_prefill_bf16_sampled():
    """Full-size batch in the benchmark's launch configuration (inference,
    no save), checked on sampled tokens: every token of the largest and of a
    few mid-size segments, plus a random sample."""
    w = gu.workload("large_prefill_bf16")
    res = gu.run(w, training=False)
    L = gu.lib()
    pl = L.l3_plan_export(res["layer"].plan)
    st = pl["seg_tok_start"]
    sizes = np.diff(st)
    order = np.argsort(-sizes, kind="stable")
    toks = [pl["perm"][st[order[0]]:st[order[0] + 1]][:256]]
    for q in (1, 10, 100, 1000):
        g = order[min(q, len(order) - 1)]
        toks.append(pl["perm"][st[g]:st[g + 1]][:32])
    rng = np.random.default_rng(0)
    toks.append(rng.choice(w.batch, 512, replace=False))
    tokens = np.unique(np.concatenate(toks))
    ref = gu.oracle_forward(w, tokens=tokens)
    _check(w, res, ref, tokens=tokens)


def test_train_skew_bf16_forward():
    w = gu.workload("train_skew_bf16")
    res = gu.run(w, training=True)
    _check(w, res, gu.oracle_forward(w))


# ------------------------------------------------------------- GPU pins ---
def test_pin_single_row_exact_fp32():
    """n_t = 1: the softmax weight is exactly 1, so a equals that V row."""
    w = gu.workload("tiny_fp32")
    res = gu.run(w, training=True)
    a = res["a32"].cpu().numpy()
    n = np.diff(w.offsets)
    hit = 0
    for i, t in enumerate(w.ids):
        if n[t] == 1:
            assert np.array_equal(a[i], w.V[w.offsets[t]])
            hit += 1
    assert hit > 0


@pytest.mark.parametrize("name", ["tiny_fp32", "train_skew_bf16"])
def test_pin_identical_keys_mean(name):
    """Identical key rows give a uniform softmax: a = mean of V_t."""
    base = gu.workload(name)
    K = base.K.copy()
    for t in range(base.spec.vocab):
        r0, r1 = base.offsets[t], base.offsets[t + 1]
        K[r0:r1] = K[r0]
    w = wl.Workload(**{**base.__dict__, "K": K})
    res = gu.run(w, training=True)
    a = gu.f64(res["a32"])
    V = wl.decode(w.V)
    want = np.stack([V[w.offsets[t]:w.offsets[t + 1]].mean(axis=0)
                     for t in w.ids])
    err = gu.max_abs(a, want)
    print(f"{name}: identical keys, max |a - mean V_t| = {err:.3e}")
    assert err <= (1e-6 if w.spec.dtype == "f32" else 2e-3)


def test_pin_row_permutation_invariance():
    """Jointly permuting each id's K and V rows leaves y unchanged."""
    base = gu.workload("tiny_fp32", True)
    rng = np.random.default_rng(3)
    K, V = base.K.copy(), base.V.copy()
    for t in range(base.spec.vocab):
        r0, r1 = base.offsets[t], base.offsets[t + 1]
        q = r0 + rng.permutation(r1 - r0)
        K[r0:r1], V[r0:r1] = base.K[q], base.V[q]
    w = wl.Workload(**{**base.__dict__, "K": K, "V": V})
    y1 = gu.f64(gu.run(base)["y"])
    y2 = gu.f64(gu.run(w)["y"])
    assert gu.linf_rel(y2, y1) <= F32_REL


def test_forward_deterministic():
    torch = gu.torch_cuda()
    w = gu.workload("prefill_bf16")
    dev = gu.Dev(w)
    y1 = gu.run(w, dev)["y"]
    y2 = gu.run(w, dev)["y"]
    assert torch.equal(y1, y2)


def test_bad_plan_makes_forward_a_noop():
    torch = gu.torch_cuda()
    L = gu.lib()
    w = gu.workload("tiny_fp32")
    dev = gu.Dev(w)
    dev.ids = dev.ids.clone()
    dev.ids[3] = w.spec.vocab + 5
    from static_token_routed_id_amd.layer import L3Layer
    layer = L3Layer(gu.desc_of(w), w.batch)
    layer.make_plan(dev.ids, dev.offsets, check_status=False)
    y = torch.full((w.batch, w.spec.d), float("nan"), device="cuda")
    layer.forward(*dev.params(), y=y)
    assert L.l3_plan_check(layer.plan) == L.L3_ERR_TOKEN_RANGE
    assert torch.isnan(y).all()


def test_empty_batch():
    torch = gu.torch_cuda()
    L = gu.lib()
    w = gu.workload("train_skew_bf16")
    dev = gu.Dev(w)
    from static_token_routed_id_amd.layer import L3Layer
    layer = L3Layer(gu.desc_of(w), 16, training=True)
    empty = torch.empty(0, dtype=torch.int32, device="cuda")
    layer.make_plan(empty, dev.offsets)
    assert layer.plan.tokens == 0
    y = layer.forward(dev.x[:0], *dev.params()[1:])
    assert y.shape == (0, w.spec.d)
    g = layer.backward(dev.dy[:0], dev.x[:0], *dev.params()[1:])
    torch.cuda.synchronize()
    for k in ("dK", "dV", "dW_up", "dgamma", "dbeta", "dW_mix"):
        assert float(g[k].abs().max()) == 0.0, k
    assert L.l3_plan_check(layer.plan) == L.L3_OK


def test_u_far_from_zero_mean():
    """LayerNorm input whose mean is tens of times its spread. Both inference
    paths keep u in bf16, and its rounding (relative to |mean|) then sets the
    error, well beyond the bf16 bound of the unshifted workloads. What is
    checked is that the folded normalisation (one-pass per-tile sums, the
    mean term cancelled against the folded weights; the 8192-token batch)
    adds nothing to it: on the same 64 tokens its rms error is within 1.5x
    of the row normalisation's (two-pass statistics of each row; the same
    tokens as a 64-token batch)."""
    w = wl.with_u_offset(gu.workload("prefill_bf16", True), 50.0)
    full = gu.f64(gu.run(w)["y"])
    tok = np.arange(64)
    w64 = wl.with_ids(w, w.ids[:64], x=np.ascontiguousarray(w.x[:64]))
    small = gu.f64(gu.run(w64)["y"])
    ref = gu.oracle_forward(w, tokens=tok)
    ratio = np.abs(ref["mean"]) / np.sqrt(ref["var"])
    e_fold = float(np.sqrt(np.mean((full[tok] - ref["y"]) ** 2)))
    e_row = float(np.sqrt(np.mean((small - ref["y"]) ** 2)))
    print(f"median |mean| / std of u {np.median(ratio):.1f}; rms error: "
          f"folded {e_fold:.3e}, row {e_row:.3e}")
    assert np.median(ratio) >= 10
    assert e_fold <= 1.5 * e_row + 1e-4


def _times8(w):
    """The workload's ids eight times over, each copy with the rows of x
    rolled by another offset (65536 tokens for the prefill shape)."""
    ids = np.concatenate([w.ids] * 8)
    x = np.ascontiguousarray(np.concatenate(
        [np.roll(w.x, 1000 * j, axis=0) for j in range(8)]))
    return wl.with_ids(w, ids, x=x)


def test_prefill_bf16_w_up_folded_sampled():
    """On large batches (here 65536 tokens of the prefill shape) inference
    folds W_up through LayerNorm into W_mix: u is never formed; each row's variance comes from a quadratic
    form of a, and y from [a ; x] against the composed weights. Checked on
    sampled tokens (both ends and a random sample) at the bf16 bound."""
    w = _times8(gu.workload("prefill_bf16"))
    assert w.batch == 65536
    res = gu.run(w, training=False)
    rng = np.random.default_rng(1)
    tokens = np.unique(np.concatenate([
        np.arange(256), rng.choice(w.batch, 1024, replace=False),
        np.arange(w.batch - 64, w.batch)]))
    ref = gu.oracle_forward(w, tokens=tokens)
    _check(w, res, ref, tokens=tokens)


def test_u_far_from_zero_mean_w_up_folded():
    """The offset input of the test above on 65536 tokens: with W_up's
    columns centred before the fold, neither the variance nor the output
    subtracts a large mean, so the error stays within 1.5x of the row
    normalisation's on the same 64 tokens (in practice well below it)."""
    w = wl.with_u_offset(_times8(gu.workload("prefill_bf16", True)), 50.0)
    full = gu.f64(gu.run(w)["y"])
    tok = np.arange(64)
    w64 = wl.with_ids(w, w.ids[:64], x=np.ascontiguousarray(w.x[:64]))
    small = gu.f64(gu.run(w64)["y"])
    ref = gu.oracle_forward(w, tokens=tok)
    ratio = np.abs(ref["mean"]) / np.sqrt(ref["var"])
    e_fused = float(np.sqrt(np.mean((full[tok] - ref["y"]) ** 2)))
    e_row = float(np.sqrt(np.mean((small - ref["y"]) ** 2)))
    print(f"median |mean| / std of u {np.median(ratio):.1f}; rms error: "
          f"W_up folded {e_fused:.3e}, row {e_row:.3e}")
    assert np.median(ratio) >= 10
    assert e_fused <= 1.5 * e_row + 1e-4
