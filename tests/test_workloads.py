"""The seeded input generators: shapes, row counts, determinism, rounding."""
import numpy as np
import pytest
import torch

from static_token_routed_id_amd import workloads as wl

# rows R = sum of capped Zipf allocations, one per configuration
EXPECTED_ROWS = {"tiny_fp32": 1135, "prefill_bf16": 171462,
                 "decode_bf16": 588017, "large_prefill_bf16": 1759242,
                 "train_skew_bf16": 1615, "train_skew_prefill_bf16": 171462}


@pytest.mark.parametrize("name", wl.CONFIG_ORDER)
def test_allocation(name):
    spec = wl.SPECS[name]
    n = wl.allocation(spec)
    assert n.min() >= 1 and n.max() <= spec.k_max
    assert int(n.sum()) == EXPECTED_ROWS[name]
    ids = wl.batch_ids(spec, wl.CONFIG_ORDER.index(name))
    assert ids.shape == (spec.batch,) and ids.dtype == np.int32
    assert ids.min() >= 0 and ids.max() < spec.vocab
    assert np.array_equal(ids, wl.batch_ids(spec, wl.CONFIG_ORDER.index(name)))


def test_hot_id_share():
    spec = wl.SPECS["train_skew_bf16"]
    ids = wl.batch_ids(spec, 4)
    assert int((ids == 0).sum()) == round(0.3 * spec.batch) == 154
    assert wl.allocation(spec)[0] == 512


def test_small_workloads_deterministic():
    a = wl.make("tiny_fp32")
    b = wl.make(0)
    for f in ("ids", "offsets", "x", "K", "V", "W_up", "W_mix"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f
    assert a.K.dtype == np.float32 and a.K.shape == (1135, 64)
    c = wl.make("train_skew_bf16")
    assert c.K.dtype == np.uint16 and c.dy.shape == (512, 64)


def test_bf16_rounding_matches_torch():
    g = np.random.default_rng(0)
    v = np.concatenate([g.standard_normal(100000).astype(np.float32),
                        np.float32([0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8,
                                    65504.0, 1e-30])])
    mine = wl.f32_to_bf16_bits(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(mine, ref.view(np.uint16))
    back = wl.bf16_bits_to_f32(mine)
    assert np.array_equal(back, torch.from_numpy(v).to(torch.bfloat16)
                          .float().numpy())


def test_u_offset_is_a_common_row():
    """with_u_offset adds the same vector to every row of W_up (up to the
    storage rounding) and leaves every other input alone."""
    w = wl.make("tiny_fp32")
    w2 = wl.with_u_offset(w, 50.0)
    diff = wl.decode(w2.W_up) - wl.decode(w.W_up)
    assert np.abs(diff - diff[0]).max() <= 1e-5 * np.abs(diff).max()
    assert np.abs(diff[0]).max() > 1.0
    assert w2.x is w.x and w2.K is w.K and w2.W_mix is w.W_mix


def _golden_sha():
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden",
                        "workload_sha256.json")
    with open(path) as f:
        return json.load(f)


def test_numpy_version_pinned():
    """The input hashes below were recorded with this numpy version (the
    generators' streams are PCG64 and standard_normal, stable by numpy's own
    policy; a different version must reproduce the hashes to be trusted)."""
    assert np.__version__ == _golden_sha()["numpy"]


@pytest.mark.parametrize("name", ["tiny_fp32", "train_skew_bf16"])
def test_generated_arrays_sha256(name):
    """Every array of the tiny forward and tiny training workloads hashes
    to the value recorded by tests/golden/make_workload_sha256.py, so a
    silent change of the generators (or of numpy's streams) shows."""
    import hashlib
    want = _golden_sha()["workloads"][name]
    w = wl.make(name)
    for f, digest in want.items():
        a = np.ascontiguousarray(getattr(w, f))
        h = hashlib.sha256()
        h.update(f"{a.dtype.str}{a.shape}".encode())
        h.update(a.tobytes())
        assert h.hexdigest() == digest, f
