"""GPU plan (sort by id + segments) against the oracle, bit for bit.

Covers every device path: the one-wavefront plan (up to 64 tokens), the
single-workgroup bitonic sort (up to 4096 tokens: in registers with one key
a thread up to 1024, in LDS above) and the multi-kernel radix
sort (larger batches, 1 to 3 digit passes of 8 or 9 bits), with batches on
both sides of each boundary."""
import numpy as np
import pytest

from oracle import l3_oracle
from static_token_routed_id_amd import workloads as wl
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _plan_and_compare(ids, offsets, vocab, k_max=512, rows=None):
    torch = gu.torch_cuda()
    L = gu.lib()
    rows = int(offsets[-1]) if rows is None else rows
    desc = L.make_desc(vocab, rows, 64, 64, k_max, L.L3_BF16)
    B = len(ids)
    p, _, _ = L.l3_workspace_size(desc, B)
    ws = torch.empty(max(p, 256), dtype=torch.uint8, device="cuda")
    d_ids = torch.from_numpy(np.ascontiguousarray(ids, np.int32)).cuda()
    d_off = torch.from_numpy(np.ascontiguousarray(offsets, np.int64)).cuda()
    print(f"plan B={B} vocab={vocab}", flush=True)
    plan = L.l3_plan(desc, d_ids, d_off, ws)
    assert L.l3_plan_check(plan) == L.L3_OK
    got = L.l3_plan_export(plan)
    want = l3_oracle.plan(ids, offsets, vocab, k_max, rows)
    assert got["S"] == want["S"]
    for k in ("perm", "seg_id", "seg_tok_start", "seg_row_off", "seg_n"):
        assert np.array_equal(got[k].astype(np.int64), want[k]), k
    return got


@pytest.mark.parametrize("name", wl.CONFIG_ORDER)
def test_plan_configs(name):
    spec = wl.SPECS[name]
    cfg = wl.CONFIG_ORDER.index(name)
    offsets = wl.offsets_from_counts(wl.allocation(spec))
    ids = wl.batch_ids(spec, cfg)
    _plan_and_compare(ids, offsets, spec.vocab)


def _offsets(vocab, seed, kmax=8):
    rng = np.random.default_rng(seed)
    return wl.offsets_from_counts(rng.integers(1, kmax + 1, vocab))


ADVERSARIAL = {
    "one_token": lambda: (np.array([5], np.int32), 50),
    "all_same_small": lambda: (np.full(3000, 7, np.int32), 50),
    "all_same_large": lambda: (np.full(20000, 7, np.int32), 50),
    "all_distinct_small": lambda: (
        np.random.default_rng(1).permutation(4096).astype(np.int32), 4096),
    "all_distinct_8192": lambda: (
        np.random.default_rng(8).permutation(8192).astype(np.int32), 8192),
    "ragged_4097": lambda: (
        np.random.default_rng(9).integers(0, 3000, 4097).astype(np.int32),
        3000),
    "all_distinct_large": lambda: (
        np.random.default_rng(2).permutation(40000).astype(np.int32), 40000),
    "max_id_only": lambda: (np.full(17, 99, np.int32), 100),
    # batches of at most 64 tokens (the one-wavefront plan)
    "two_tokens_same": lambda: (np.array([9, 9], np.int32), 50),
    "two_tokens_reversed": lambda: (np.array([30, 2], np.int32), 50),
    "all_same_64": lambda: (np.full(64, 3, np.int32), 50),
    "reverse_sorted_64": lambda: (np.arange(64)[::-1].astype(np.int32).copy(),
                                  64),
    "repeats_33": lambda: (
        np.random.default_rng(12).integers(0, 5, 33).astype(np.int32), 5),
    "ragged_63": lambda: (
        np.random.default_rng(13).integers(0, 40, 63).astype(np.int32), 40),
    "presorted_large": lambda: (
        np.sort(np.random.default_rng(3).integers(0, 5000, 30000))
        .astype(np.int32), 5000),
    "reverse_sorted_large": lambda: (
        np.sort(np.random.default_rng(4).integers(0, 5000, 30000))[::-1]
        .astype(np.int32).copy(), 5000),
    # 65 .. 1024 tokens (the single-workgroup sort with one key a thread)
    "ragged_65": lambda: (
        np.random.default_rng(17).integers(0, 30, 65).astype(np.int32), 30),
    "ragged_513": lambda: (
        np.random.default_rng(18).integers(0, 700, 513).astype(np.int32),
        700),
    "reverse_sorted_1000": lambda: (
        np.sort(np.random.default_rng(19).integers(0, 400, 1000))[::-1]
        .astype(np.int32).copy(), 400),
    "all_same_1024": lambda: (np.full(1024, 11, np.int32), 50),
    # 4097 .. 8192 tokens: the radix sort on few tiles
    "all_same_8192": lambda: (np.full(8192, 7, np.int32), 50),
    "reverse_sorted_7777": lambda: (
        np.sort(np.random.default_rng(14).integers(0, 5000, 7777))[::-1]
        .astype(np.int32).copy(), 5000),
    "three_digit_passes_8000": lambda: (
        np.random.default_rng(15).integers(0, 1 << 20, 8000)
        .astype(np.int32), 1 << 20),
    "two_nine_bit_passes_6001": lambda: (
        np.random.default_rng(16).integers(0, 1 << 17, 6001)
        .astype(np.int32), 1 << 17),
    "ragged_8193": lambda: (
        np.random.default_rng(5).integers(0, 3000, 8193).astype(np.int32),
        3000),
    "one_digit_pass_large": lambda: (
        np.random.default_rng(6).integers(0, 200, 50000).astype(np.int32),
        200),
    "three_digit_passes": lambda: (
        np.random.default_rng(7).integers(0, 1 << 20, 100000)
        .astype(np.int32), 1 << 20),
}


@pytest.mark.parametrize("case", sorted(ADVERSARIAL))
def test_plan_adversarial(case):
    ids, vocab = ADVERSARIAL[case]()
    _plan_and_compare(ids, _offsets(vocab, 11), vocab, k_max=8)


def test_plan_hot_id_at_cap():
    vocab = 300
    counts = np.random.default_rng(8).integers(1, 33, vocab)
    counts[0] = 512
    offsets = wl.offsets_from_counts(counts)
    ids = np.random.default_rng(9).integers(0, vocab, 5000).astype(np.int32)
    ids[::3] = 0
    _plan_and_compare(ids, offsets, vocab, k_max=512)


@pytest.mark.parametrize("B", [50, 64, 100, 6000, 12000])
def test_plan_errors(B):
    torch = gu.torch_cuda()
    L = gu.lib()
    vocab = 64
    counts = np.full(vocab, 4)
    counts[10] = 0      # id 10 owns no row
    counts[20] = 9      # id 20 owns more than k_max = 8 rows
    offsets = wl.offsets_from_counts(counts)
    desc = L.make_desc(vocab, int(offsets[-1]), 64, 64, 8, L.L3_BF16)
    p, _, _ = L.l3_workspace_size(desc, B)
    ws = torch.empty(p, dtype=torch.uint8, device="cuda")
    d_off = torch.from_numpy(offsets).cuda()
    rng = np.random.default_rng(B)
    cases = [
        (np.where(np.arange(B) == B // 2, vocab, 3), L.L3_ERR_TOKEN_RANGE),
        (np.where(np.arange(B) == 1, -1, 3), L.L3_ERR_TOKEN_RANGE),
        (np.where(np.arange(B) == 7, 10, 3), L.L3_ERR_COUNT),
        (np.where(np.arange(B) == 5, 20, 3), L.L3_ERR_COUNT),
        # both kinds at once: the id range is reported first, on every path
        (np.where(np.arange(B) == B - 1, vocab + 5,
                  np.where(np.arange(B) == 7, 10, 3)), L.L3_ERR_TOKEN_RANGE),
        (rng.integers(0, 10, B), L.L3_OK),
    ]
    for ids, want in cases:
        d_ids = torch.from_numpy(ids.astype(np.int32)).cuda()
        print(f"plan error case B={B} want={want}", flush=True)
        plan = L.l3_plan(desc, d_ids, d_off, ws, check_status=False)
        assert L.l3_plan_check(plan) == want
