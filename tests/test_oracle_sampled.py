"""The sampled whole-batch reference of the training parity test at full
size (tests/gpu_util.oracle_backward_sampled) against the oracle's own
backward, on a small training workload where the latter is cheap: every
token and every id sampled, all seven gradients equal to float64 rounding.
"""
import dataclasses

import numpy as np
import pytest

from static_token_routed_id_amd import workloads as wl
from tests import gpu_util as gu


@pytest.mark.parametrize("chunk", [1024, 64])
def test_sampled_reference_equals_oracle_backward(chunk):
    """chunk 64: ids spread over several chunks on four threads, so an id's
    dK / dV adds partial sums from several workers."""
    w = wl.make("train_skew_bf16")
    w = dataclasses.replace(w, dy=wl.upstream_grad(w))
    B = w.batch
    present = np.unique(w.ids)
    ref = gu.oracle_backward(w)
    got = gu.oracle_backward_sampled(w, range(B), present, threads=4,
                                     chunk=chunk)
    for k in ("dW_mix", "dW_up", "dgamma", "dbeta"):
        np.testing.assert_allclose(got[k], ref[k], rtol=1e-10, atol=1e-10)
    for i in range(B):
        np.testing.assert_allclose(got["dx"][i], ref["dx"][i], rtol=1e-10,
                                   atol=1e-10)
    for t in present:
        r0, r1 = int(w.offsets[t]), int(w.offsets[t + 1])
        np.testing.assert_allclose(got["dK"][int(t)], ref["dK"][r0:r1],
                                   rtol=1e-10, atol=1e-10)
        np.testing.assert_allclose(got["dV"][int(t)], ref["dV"][r0:r1],
                                   rtol=1e-10, atol=1e-10)
