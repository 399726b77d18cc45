"""Benchmark of the L3 layer forward on one MI355X.

One step = plan (sort by id, segments, work items) + forward (segment
softmax-aggregate, W_up projection, LayerNorm, W_mix projection) of one
batch, all resident in HBM before timing starts. Default workload: the
large-prefill configuration (65536 tokens, vocab 131072, 2^22-row budget,
d = 2048, d_e = 512, bf16 inputs, float32 accumulation and output).
`--train` times a training step instead: plan + forward keeping the saved
state + backward with a seeded upstream gradient (fwd+bwd tokens/s, every
stage's mean ms), e.g. `--train --workload train_skew_bf16`. `--offload
--workload decode_bf16` keeps the tables in pinned host memory and stages
the batch's rows into HBM beside a stand-in for the preceding layers,
against the same step with the tables in HBM. `--allocate` times the
embedding allocation (host code) on a synthetic corpus. `--layers L`
times plan + L layer forwards (each layer its own tables and weights over
the same offsets, one plan for the stack): tokens/s through the stack.

Prints one JSON line. `roofline` is the gather/aggregate step: on large
bf16 batches one launch of seg_group_kernel (it also runs the wave items of
the ids with few rows), else seg_fwd_kernel (+ seg_combine for split rows):
algorithmic bytes per launch (each distinct id's K_t and V_t rows once, x
read, a written, ids and segment records) over the mean launch time, taken
from HIP events the library records on the launch stream around each
stage in a second run of as many steps (the headline steps run without
those events); `traffic` is the HBM bytes per launch from the committed
FETCH_SIZE / WRITE_SIZE counter summary
(profiles/traffic_gather_<workload>.md), or null when the kernels changed
since it was taken; `copy_peak_gbs` is a measured 2 GiB device copy (bytes
read + written per second) and `frac_of_copy_peak` the gather's rate
against it (above 1: the gather mostly reads); `read_peak_gbs` are reads
of a 4 GiB buffer by the read probe (libl3probe.so) in the gather's own
access pattern, contiguous, and contiguous non-temporal, with
`frac_of_read_peak` the gather's algorithmic rate against the first and
`traffic_rate_gbs` its counter-measured HBM bytes per second. `cpu_baseline` is the fp64 oracle on a bounded sample of the
same batch on the host CPU (one oracle call per host thread, CPU model
recorded). Workloads whose step moves less than 1 GiB (everything but the
large prefill) are timed step by step with HIP events, L2 and the MALL
flushed between steps by a 1 GiB write outside the events (`--flush`).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "L3 layer fwd tokens/sec + achieved HBM GB/s of K/V gather vs peak, bf16"
METRIC_TRAIN = "L3 layer fwd+bwd tokens/sec (training step) + per-stage ms"
METRIC_STACK = "L3 stack fwd tokens/sec (one plan shared by every layer)"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 MFMA


def algorithmic_bytes(w, plan, group_min_rows: int) -> dict:
    """Bytes the gather/aggregate step must move, per launch, split by the
    kernel that handles each id: every distinct id's K_t and V_t rows once,
    its tokens' x rows read and a rows written, the token index and the
    segment record."""
    e = 2 if w.spec.dtype == "bf16" else 4
    d, d_e = w.spec.d, w.spec.d_e
    n = np.asarray(plan["seg_n"], np.int64)
    m = np.diff(np.asarray(plan["seg_tok_start"], np.int64))
    per_seg = n * (d + d_e) * e + m * (d * e + d_e * e + 4) + 16
    grp = (n >= group_min_rows) if group_min_rows > 0 else np.zeros_like(n, bool)
    out = dict(group=int(per_seg[grp].sum()), wave=int(per_seg[~grp].sum()))
    out["total"] = out["group"] + out["wave"]
    out["table"] = int((n * (d + d_e) * e).sum())
    return out


# Sources whose change invalidates the committed HBM traffic counts of the
# gather kernels (kernel code, shared device helpers, launch configuration,
# and the plan, whose item lists set the order the items run in).
TRAFFIC_SOURCES = ("static_token_routed_id_amd/csrc/seg_fwd.hip",
                   "static_token_routed_id_amd/csrc/seg_group.hip",
                   "static_token_routed_id_amd/csrc/seg_wave.h",
                   "static_token_routed_id_amd/csrc/l3_device.h",
                   "static_token_routed_id_amd/csrc/l3_internal.h",
                   "static_token_routed_id_amd/csrc/api.cpp",
                   "static_token_routed_id_amd/csrc/plan.hip")


def sources_digest() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(rel.encode() + b"\0" + f.read() + b"\0")
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch of the gather kernels from the committed
    FETCH_SIZE / WRITE_SIZE counter summary of this workload, or None when
    there is none or the kernels changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_gather_{workload}.md")
    try:
        text = open(path).read()
    except OSError:
        return None
    start = text.find("```json")
    if start < 0:
        return None
    end = text.find("```", start + 7)
    try:
        rec = json.loads(text[start + 7:end])
    except ValueError:
        return None
    if rec.get("sources_digest") != sources_digest():
        return None
    return rec


def calibrate_copy(nbytes: int = 1 << 30, reps: int = 3) -> None:
    """A plain device-to-device copy of known size, the reference launch for
    scaling the FETCH_SIZE / WRITE_SIZE counters to bytes."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes,
                      "reps": reps}), flush=True)


def gemm_flops(w) -> dict:
    B, d, d_e = w.batch, w.spec.d, w.spec.d_e
    # up_quad / mix_up_proj: the forward with W_up folded into W_mix (a G
    # over K = 2 d_e for the row variances, [a ; x] over K = d_e + d)
    return dict(up_proj=2.0 * B * d * d_e, mix_proj=2.0 * B * d * 2 * d,
                up_quad=2.0 * B * d_e * 2 * d_e,
                mix_up_proj=2.0 * B * d * (d_e + d))


def cpu_baseline_train(w, dy, budget_s: float) -> dict:
    """The oracle's forward + backward (as it stands) on a bounded sample of
    the batch (the first n tokens as a batch of their own), or None when its
    dense float64 dK would not fit comfortably in host memory."""
    from threadpoolctl import threadpool_limits

    from oracle import l3_oracle
    from static_token_routed_id_amd import workloads as wl
    if w.rows * w.spec.d * 8 > (4 << 30):
        return None
    dd = wl.decoded(w)
    dyd = wl.decode(dy)

    def run(n):
        args = [dd["x"][:n], dd["ids"][:n], dd["K"], dd["V"], dd["offsets"],
                dd["W_up"], dd["gamma"], dd["beta"], dd["W_mix"]]
        t0 = time.perf_counter()
        l3_oracle.forward(*args)
        l3_oracle.backward(*args, dyd[:n])
        return time.perf_counter() - t0

    with threadpool_limits(limits=1):
        n = min(w.batch, 16)
        dt = run(n)
        n = int(min(w.batch, max(16, budget_s / max(dt / n, 1e-6))))
        dt = run(n)
    return {"value": n / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "cpu": cpu_model(),
            "sample": f"the first {n} tokens of the {w.batch}-token batch as "
                      f"a batch of their own, forward and backward in "
                      f"float64, one thread, {dt:.1f} s"}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_threads() -> int:
    """Host threads for the oracle baseline: the CPUs this process may run
    on, at most 16 (a one-GPU share of the host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline(w, budget_s: float) -> dict:
    """The oracle (as it stands) on a bounded sample of the batch: the
    sampled tokens split into one slice per host thread, each slice one
    oracle.forward call (tokens are independent), BLAS single-threaded
    inside each call; wall time of the whole sample."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    from oracle import l3_oracle
    from static_token_routed_id_amd import workloads as wl
    dd = wl.decoded(w)
    args = [dd[k] for k in ("x", "ids", "K", "V", "offsets", "W_up", "gamma",
                            "beta", "W_mix")]
    rng = np.random.default_rng(1234)
    order = rng.permutation(w.batch)
    T = cpu_threads()

    def run(n):
        parts = np.array_split(order[:n], T)
        t0 = time.perf_counter()
        with ThreadPoolExecutor(T) as ex:
            list(ex.map(lambda tk: l3_oracle.forward(*args, tokens=tk),
                        [p for p in parts if len(p)]))
        return time.perf_counter() - t0

    with threadpool_limits(limits=1):
        n = min(w.batch, 16 * T)
        dt = run(n)
        n = int(min(w.batch, max(n, budget_s / max(dt / n, 1e-6))))
        dt = run(n)
    return {"value": n / dt, "unit": "tokens/s", "cores": T, "kind": "oracle",
            "cpu": cpu_model(),
            "sample": f"{n} tokens drawn at random (seed 1234) from the "
                      f"{w.batch}-token batch, full layer forward in float64, "
                      f"{T} threads (one oracle.forward call per thread on "
                      f"its share of the sample), {dt:.1f} s wall"}


def copy_peak_gbs(nbytes: int = 1 << 31, reps: int = 5) -> float:
    """Measured device-copy rate (bytes read + written per second) of a
    2 GiB device-to-device copy, the practical HBM ceiling beside the 8 TB/s
    of the data sheet."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    src.fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(
        enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    del src, dst
    return 2 * nbytes / (ms * 1e-3) / 1e9


def read_peak_gbs(nbytes: int = 1 << 32, reps: int = 5) -> dict:
    """Measured read rates (GB/s, best over three grid sizes) of a 4 GiB
    device buffer streamed by the read probe (csrc/read_probe.hip,
    libl3probe.so): the gather's own access pattern (16 rows of 4 KiB a
    64 KiB block, 64 bytes of each row per wave instruction), 1 KiB
    contiguous per instruction, the same with non-temporal loads, and the
    gather's pattern with non-temporal loads (the two halves of each
    128-byte line read by consecutive instructions, or four apart)."""
    import ctypes

    import torch
    from static_token_routed_id_amd import build as B
    if not os.path.exists(B.PROBE_LIB):
        raise RuntimeError(f"{B.PROBE_LIB} is not built: run "
                           "python -m static_token_routed_id_amd.build")
    lib = ctypes.CDLL(B.PROBE_LIB)
    lib.l3probe_read.argtypes = [ctypes.c_void_p, ctypes.c_int64,
                                 ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                 ctypes.c_void_p]
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(7)
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream()
    out = {}
    for name, pattern in (("gather_pattern", 1), ("stream", 0),
                          ("stream_nontemporal", 2),
                          ("gather_pattern_nontemporal", 3),
                          ("gather_pattern_nontemporal_halves_apart", 4)):
        best = 0.0
        for grid in (512, 1024, 2048):
            def launch():
                rc = lib.l3probe_read(buf.data_ptr(), nbytes, pattern, grid,
                                      sink.data_ptr(), st.cuda_stream)
                if rc != 0:
                    raise RuntimeError(f"l3probe_read returned {rc}")
            launch()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(
                enable_timing=True)
            a.record(st)
            for _ in range(reps):
                launch()
            b.record(st)
            torch.cuda.synchronize()
            best = max(best, nbytes / (a.elapsed_time(b) / reps * 1e-3) / 1e9)
        out[name] = round(best, 1)
    del buf
    return out


def run_offload(args) -> None:
    """Decode with the tables in pinned host memory: per step the plan, then
    the batch's rows staged into HBM on a side stream while a stand-in for
    the preceding layers (bf16 GEMMs streaming --prelayer-gb of weights)
    runs on the main stream, then the layer's forward on the staged rows.
    Compared with the same step with the tables in HBM."""
    import torch

    from static_token_routed_id_amd import _lib as L
    from static_token_routed_id_amd import workloads as wl
    from static_token_routed_id_amd.layer import L3Layer, to_device

    w = wl.make(args.workload)
    dtype = L.L3_BF16 if w.spec.dtype == "bf16" else L.L3_F32
    desc = L.make_desc(w.spec.vocab, w.rows, w.spec.d, w.spec.d_e,
                       w.spec.k_max, dtype, L.L3_F32)
    dev = {k: to_device(getattr(w, k)) for k in
           ("x", "K", "V", "W_up", "gamma", "beta", "W_mix")}

    def pinned(a):
        if a.dtype == np.uint16:
            t = torch.from_numpy(np.ascontiguousarray(a.view(np.int16)))
            return t.pin_memory().view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).pin_memory()

    K_host, V_host = pinned(w.K), pinned(w.V)
    ids = torch.from_numpy(w.ids).cuda()
    offsets = torch.from_numpy(w.offsets).cuda()
    B, d, d_e = w.batch, w.spec.d, w.spec.d_e
    stage_rows = min(w.rows, B * w.spec.k_max)
    tdt = dev["K"].dtype
    K_stage = torch.empty((stage_rows, d), dtype=tdt, device="cuda")
    V_stage = torch.empty((stage_rows, d_e), dtype=tdt, device="cuda")
    u = np.unique(w.ids)
    rows = int((w.offsets[u + 1] - w.offsets[u]).sum())
    stage_bytes = rows * (d + d_e) * (2 if w.spec.dtype == "bf16" else 4)
    # stand-in for the layers before this one: weight-streaming GEMMs
    width = 4096
    n_w = max(1, int(args.prelayer_gb * 1e9 / (2 * width * 8192)))
    W_pre = [torch.randn(width, 8192, device="cuda").to(torch.bfloat16)
             for _ in range(n_w)]
    x_pre = torch.randn(B, width, device="cuda").to(torch.bfloat16)

    def prelayers():
        for Wp in W_pre:
            torch.mm(x_pre, Wp)

    layer = L3Layer(desc, B)
    y = torch.empty((B, d), dtype=torch.float32, device="cuda")
    params = [dev[k] for k in ("x", "K", "V", "W_up", "gamma", "beta",
                               "W_mix")]
    staged = [dev["x"], K_stage, V_stage, dev["W_up"], dev["gamma"],
              dev["beta"], dev["W_mix"]]
    side = torch.cuda.Stream()
    main_s = torch.cuda.current_stream()

    def step_hbm():
        layer.make_plan(ids, offsets)
        prelayers()
        layer.forward(*params, y=y)

    def step_offload():
        layer.make_plan(ids, offsets)
        side.wait_stream(main_s)
        with torch.cuda.stream(side):
            L.l3_stage_rows(layer.plan, K_host, V_host, K_stage, V_stage,
                            stream=side)
        prelayers()
        main_s.wait_stream(side)
        layer.forward(*staged, y=y)

    plan_done = torch.cuda.Event()

    def step_offload_dma():
        # the stand-in is queued before the host waits for the plan, so the
        # GPU never idles while the copies are queued
        layer.make_plan(ids, offsets)
        plan_done.record(main_s)
        prelayers()
        side.wait_event(plan_done)
        L.l3_stage_rows(layer.plan, K_host, V_host, K_stage, V_stage,
                        stream=side, dma=True)
        main_s.wait_stream(side)
        layer.forward(*staged, y=y)

    def step_stage_only():
        layer.make_plan(ids, offsets)
        L.l3_stage_rows(layer.plan, K_host, V_host, K_stage, V_stage)

    def step_stage_dma_only():
        layer.make_plan(ids, offsets)
        L.l3_stage_rows(layer.plan, K_host, V_host, K_stage, V_stage,
                        dma=True)

    def step_pre_only():
        prelayers()

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / args.steps

    ms_hbm = timed(step_hbm)
    ms_off_k = timed(step_offload)
    ms_off = timed(step_offload_dma)
    ms_stage_k = timed(step_stage_only)
    ms_stage = timed(step_stage_dma_only)
    ms_pre = timed(step_pre_only)
    layer.make_plan(ids, offsets)
    L.l3_stage_rows(layer.plan, K_host, V_host, K_stage, V_stage)
    assert L.l3_plan_check(layer.plan) == L.L3_OK
    out = {
        "metric": "L3 decode step with tables in pinned host memory (rows "
                  "staged beside the preceding layers) vs tables in HBM",
        "value": round(B / (ms_off * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_off, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.spec.dtype,
        "data": "synthetic (seeded Zipf ids and allocation, Gaussian tables "
                "and weights)",
        "config": {"workload": w.spec.name, "tokens": B,
                   "table_rows": w.rows, "d": d, "d_e": d_e,
                   "step": "plan + preceding-layer stand-in + forward",
                   "prelayer_weight_gb": round(n_w * 2 * width * 8192 / 1e9,
                                               2)},
        "offload": {
            "ms_step_tables_in_hbm": round(ms_hbm, 4),
            "ms_step_tables_in_host": round(ms_off, 4),
            "overhead_frac": round(ms_off / ms_hbm - 1.0, 4),
            "staging": "DMA engines (l3_stage_rows_dma)",
            "ms_step_tables_in_host_copy_kernel": round(ms_off_k, 4),
            "overhead_frac_copy_kernel": round(ms_off_k / ms_hbm - 1.0, 4),
            "ms_stage_alone": round(ms_stage, 4),
            "ms_stage_alone_copy_kernel": round(ms_stage_k, 4),
            "ms_prelayers_alone": round(ms_pre, 4),
            "staged_rows": rows,
            "staged_bytes": stage_bytes,
            "host_link_GBs": round(stage_bytes / (ms_stage * 1e-3) / 1e9, 1),
        },
    }
    print(json.dumps(out), flush=True)


def run_allocate(args) -> None:
    """The embedding allocation (host code): l3_allocate's LZW-variant scan
    of a seeded synthetic corpus at the large prefill's allocation shape
    (vocab 131072, budget 2^22 rows, k = 512), against the oracle's scan of
    a prefix of the same corpus; the uniform split beside it."""
    from static_token_routed_id_amd import _lib as L
    from static_token_routed_id_amd import workloads as wl
    spec = wl.SPECS["large_prefill_bf16"]
    V, budget, k = spec.vocab, spec.budget, spec.k_max
    n = int(args.corpus_tokens)
    t0 = time.perf_counter()
    corpus = wl.synthetic_corpus(V, n, seed=1)
    gen_s = time.perf_counter() - t0
    for _ in range(max(0, args.warmup)):
        L.l3_allocate(L.L3_ALLOC_LZW, corpus, V, budget, k)
    reps = max(1, args.steps)
    t0 = time.perf_counter()
    for _ in range(reps):
        counts, offsets = L.l3_allocate(L.L3_ALLOC_LZW, corpus, V, budget, k)
    dt = (time.perf_counter() - t0) / reps
    # tokens the scan read before the budget ran out: the prefix whose own
    # scan reaches the same rows
    t0 = time.perf_counter()
    ucounts, _ = L.l3_allocate(L.L3_ALLOC_UNIFORM, None, V, budget, k)
    dt_u = time.perf_counter() - t0
    out = {
        "metric": "embedding allocation corpus tokens/s (LZW-variant scan, "
                  "host)",
        "value": round(n / dt, 1), "unit": "tokens/s", "n_gpus": 0,
        "steps": reps, "warmup": args.warmup,
        "ms_per_step": round(dt * 1e3, 3), "higher_is_better": True,
        "vs_baseline": None, "dtype": "int32",
        "data": "synthetic corpus (seeded Zipf phrase book, Zipf phrase "
                "draws)",
        "config": {"workload": "allocation of the large prefill",
                   "vocab": V, "budget": budget, "k_max": k,
                   "corpus_tokens": n, "corpus_gen_s": round(gen_s, 2)},
        "allocation": {"rows": int(counts.sum()),
                       "max": int(counts.max()),
                       "at_cap": int((counts == k).sum()),
                       "at_one": int((counts == 1).sum()),
                       "median": float(np.median(counts)),
                       "top_1pct_share": round(float(
                           np.sort(counts)[::-1][:V // 100].sum()
                           / counts.sum()), 4)},
        "uniform": {"rows": int(ucounts.sum()), "ms": round(dt_u * 1e3, 3)},
    }
    if args.cpu_seconds > 0:
        from oracle import allocation as A
        m = min(n, 200_000)
        t0 = time.perf_counter()
        A.lzw(corpus[:m], V, budget, k)
        dto = time.perf_counter() - t0
        m = int(min(n, max(m, args.cpu_seconds / max(dto / m, 1e-9))))
        t0 = time.perf_counter()
        ref = A.lzw(corpus[:m], V, budget, k)
        dto = time.perf_counter() - t0
        same, _ = L.l3_allocate(L.L3_ALLOC_LZW, corpus[:m], V, budget, k)
        out["cpu_baseline"] = {
            "value": m / dto, "unit": "tokens/s", "cores": 1,
            "kind": "oracle", "cpu": cpu_model(),
            "sample": f"the first {m} corpus tokens, pure-Python scan, one "
                      f"thread, {dto:.1f} s (library result on the same "
                      f"prefix identical: {bool(np.array_equal(same, ref))})"}
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="large_prefill_bf16")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="time budget of the oracle baseline (0 = skip)")
    ap.add_argument("--train", action="store_true",
                    help="time plan + saving forward + backward instead")
    ap.add_argument("--layers", type=int, default=1,
                    help="forward a stack of this many layers (own tables "
                         "and weights, same offsets) with one plan a step")
    ap.add_argument("--offload", action="store_true",
                    help="decode with the tables in pinned host memory, "
                         "their rows staged beside a stand-in for the "
                         "preceding layers (use with --workload decode_bf16)")
    ap.add_argument("--prelayer-gb", type=float, default=5.2,
                    help="weights the preceding-layer stand-in streams a step "
                         "(5.2 GB: a 2.6B-parameter model in bf16)")
    ap.add_argument("--allocate", action="store_true",
                    help="time the embedding allocation (host) instead")
    ap.add_argument("--corpus-tokens", type=float, default=16e6,
                    help="synthetic corpus length for --allocate")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a 1 GiB device copy (counter calibration)")
    ap.add_argument("--flush", choices=("auto", "on", "off"), default="auto",
                    help="flush L2 and MALL between timed steps (auto: when "
                         "a step's algorithmic bytes are under 1 GiB)")
    ap.add_argument("--no-copy-peak", dest="copy_peak", action="store_false",
                    help="skip the measured device-copy and read rates")
    args = ap.parse_args()
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not "
              "supported (this build runs on a single MI355X)",
              file=sys.stderr)
        sys.exit(2)
    if args.offload:
        run_offload(args)
        return
    if args.allocate:
        run_allocate(args)
        return

    import torch

    from static_token_routed_id_amd import _lib as L
    from static_token_routed_id_amd import workloads as wl
    from static_token_routed_id_amd.layer import L3Layer, to_device

    t_gen = time.time()
    w = wl.make(args.workload)
    print(f"# generated {args.workload} in {time.time() - t_gen:.1f} s",
          file=sys.stderr, flush=True)
    dtype = L.L3_BF16 if w.spec.dtype == "bf16" else L.L3_F32
    desc = L.make_desc(w.spec.vocab, w.rows, w.spec.d, w.spec.d_e,
                       w.spec.k_max, dtype, L.L3_F32)
    if args.layers < 1 or (args.layers > 1 and args.train):
        print("--layers takes a positive count, without --train",
              file=sys.stderr)
        sys.exit(2)
    dev = {k: to_device(getattr(w, k)) for k in
           ("x", "K", "V", "W_up", "gamma", "beta", "W_mix")}
    stack = []
    for li in range(1, args.layers):
        wl_i = wl.layer_params(w, li)
        stack.append([dev["x"]] + [to_device(getattr(wl_i, k)) for k in
                                   ("K", "V", "W_up")] +
                     [dev["gamma"], dev["beta"], to_device(wl_i.W_mix)])
        del wl_i
    ids = torch.from_numpy(w.ids).cuda()
    offsets = torch.from_numpy(w.offsets).cuda()
    params = [dev[k] for k in ("x", "K", "V", "W_up", "gamma", "beta",
                               "W_mix")]
    layer = L3Layer(desc, w.batch, training=args.train)
    y = torch.empty((w.batch, w.spec.d), dtype=torch.float32, device="cuda")
    layer.make_plan(ids, offsets)
    assert L.l3_plan_check(layer.plan) == L.L3_OK
    plan_np = L.l3_plan_export(layer.plan)
    info = L.l3_plan_info(layer.plan)
    if args.train:
        dy_np = wl.upstream_grad(w)
        dy = to_device(dy_np)
        f32 = dict(dtype=torch.float32, device="cuda")
        d, d_e = w.spec.d, w.spec.d_e
        grads = [torch.empty((w.batch, d), **f32),
                 torch.empty((w.rows, d), **f32),
                 torch.empty((w.rows, d_e), **f32),
                 torch.empty((d, d_e), **f32), torch.empty(d, **f32),
                 torch.empty(d, **f32), torch.empty((d, 2 * d), **f32)]

    def step():
        layer.make_plan(ids, offsets)
        layer.forward(*params, y=y)
        for p_i in stack:
            layer.forward(*p_i, y=y)
        if args.train:
            L.l3_backward(layer.plan, dy, *params, layer.save, *grads,
                          layer.scratch)

    # Cache honesty: a step that touches less than the 256 MB MALL plus the
    # L2s could be served from cache by the step before; unless its
    # algorithmic bytes exceed 1 GiB, a 1 GiB write between steps (outside
    # the timed events) evicts both, and steps are timed one by one.
    ab_table = algorithmic_bytes(w, plan_np, info["group_min_rows"])["total"]
    flush = args.flush == "on" or (args.flush == "auto" and
                                   ab_table < (1 << 30))
    flush_buf = (torch.empty(1 << 28, dtype=torch.float32, device="cuda")
                 if flush else None)

    def timed_steps():
        """K steps, timed as a whole (or step by step with a flush between,
        outside the events); returns the seconds they took."""
        if flush:
            evs = [(torch.cuda.Event(enable_timing=True),
                    torch.cuda.Event(enable_timing=True))
                   for _ in range(args.steps)]
            for a_ev, b_ev in evs:
                flush_buf.fill_(float(len(evs)))
                a_ev.record()
                step()
                b_ev.record()
            torch.cuda.synchronize()
            return sum(a_ev.elapsed_time(b_ev) for a_ev, b_ev in evs) * 1e-3
        t_a = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        return time.perf_counter() - t_a

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # the headline steps run without the library's stage events; the same
    # number of steps then runs again with them, for the per-stage times
    # (and the gather's launch time of the roofline)
    L.l3_timing_enable(layer.plan, False)
    L.l3_timing_read(layer.plan)          # drop warm-up events
    torch.cuda.synchronize()
    t0, t1 = 0.0, timed_steps()
    L.l3_timing_enable(layer.plan, True)
    torch.cuda.synchronize()
    staged_s = timed_steps()
    L.l3_timing_enable(layer.plan, False)
    stages = L.l3_timing_read(layer.plan)
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    value = w.batch * args.steps / (t1 - t0)

    ab = algorithmic_bytes(w, plan_np, info["group_min_rows"])
    stage_avg = {k: (v[0] / v[1] if v[1] else 0.0) for k, v in stages.items()
                 if v[1]}
    # the gather/aggregate step: one group-kernel launch on large bf16
    # batches (it takes the wave items too), else the wave kernel (+ the
    # row-chunk combine)
    t_wave = stage_avg.get("seg_fwd", 0.0) + stage_avg.get("seg_combine", 0.0)
    t_group = stage_avg.get("seg_group", 0.0)
    gather_ms = t_wave + t_group
    achieved = ab["total"] / (gather_ms * 1e-3) / 1e9
    gbs = lambda b, t: round(b / (t * 1e-3) / 1e9, 1) if t > 0 else None
    fl = gemm_flops(w)
    mfma = {}
    for k in ("up_proj", "mix_proj", "up_quad", "mix_up_proj"):
        if k in stage_avg and stage_avg[k] > 0:
            tf = fl[k] / (stage_avg[k] * 1e-3) / 1e12
            mfma[k] = {"tflops": round(tf, 1),
                       "frac_of_bf16_peak": round(tf / MFMA_BF16_PEAK_TFS, 4)}
    # The W_up + W_mix stage as a whole, against its algorithmic flops
    # (2 B d d_e for W_up, 4 B d^2 for W_mix: the formula's projections),
    # whatever the kernels execute: with W_up folded into W_mix the stage is
    # the weight products, a G with the variance epilogue, the rstd pass and
    # W_mix over [a ; x]; otherwise W_up, LayerNorm and W_mix.
    stage_keys = ([k for k in ("weight_fold", "up_quad", "layernorm",
                               "mix_up_proj") if k in stage_avg]
                  if "mix_up_proj" in stage_avg else
                  [k for k in ("up_proj", "layernorm", "mix_proj")
                   if k in stage_avg])
    if stage_keys and not args.train:
        st_ms = sum(stage_avg[k] for k in stage_keys)
        alg = fl["up_proj"] + fl["mix_proj"]
        tf = alg / (st_ms * 1e-3) / 1e12
        mfma["up_mix_stage"] = {
            "algorithmic_gflop": round(alg / 1e9, 1), "ms": round(st_ms, 4),
            "stages": stage_keys, "tflops": round(tf, 1),
            "frac_of_bf16_peak": round(tf / MFMA_BF16_PEAK_TFS, 4)}
    traffic = measured_traffic(w.spec.name)
    out = {
        "metric": (METRIC_TRAIN if args.train else
                   METRIC_STACK if args.layers > 1 else METRIC),
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.spec.dtype,
        "data": "synthetic (seeded Zipf ids and allocation, Gaussian tables "
                "and weights)",
        "config": {"workload": w.spec.name, "tokens": w.batch,
                   "vocab": w.spec.vocab, "table_rows": w.rows,
                   "d": w.spec.d, "d_e": w.spec.d_e, "k_max": w.spec.k_max,
                   "distinct_ids": int(plan_np["S"]),
                   "step": "plan + forward (saved state) + backward"
                           if args.train else
                           f"plan + {args.layers} layer forwards"
                           if args.layers > 1 else "plan + forward"},
        "roofline": {"kernel": "gather (seg_group_kernel)" if t_group > 0
                               else "gather (seg_fwd_kernel)",
                     "bound": "hbm",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic["bytes_per_launch"] if traffic
                                else None,
                     "algorithmic_bytes_per_launch": ab["total"],
                     "avg_launch_ms": round(gather_ms, 4),
                     "bytes_by_item_kind": {"wave_items": ab["wave"],
                                            "group_items": ab["group"]}},
        "plan_info": info,
        "stage_ms": {k: round(v, 4) for k, v in stage_avg.items()},
        "mfma": mfma,
        "timing": ("HIP events around each step, L2 and MALL flushed "
                   "between steps by a 1 GiB write outside the events"
                   if flush else
                   "wall clock over the timed steps, synchronised on both "
                   "sides (no flush: a step touches far more than the "
                   "caches hold)") +
                  "; stage_ms from the library's per-stage HIP events in a "
                  "second run of as many steps (%.4f ms a step with the "
                  "events), the headline steps run without them"
                  % (staged_s * 1e3 / args.steps),
    }
    if args.copy_peak:
        cp = copy_peak_gbs()
        out["roofline"]["copy_peak_gbs"] = round(cp, 1)
        out["roofline"]["frac_of_copy_peak"] = round(achieved / cp, 4)
        rp = read_peak_gbs()
        out["roofline"]["read_peak_gbs"] = rp
        out["roofline"]["frac_of_read_peak"] = round(
            achieved / rp["gather_pattern"], 4)
        if traffic:
            # counter-measured HBM bytes a launch over its time
            hbm = traffic["bytes_per_launch"] / (gather_ms * 1e-3) / 1e9
            out["roofline"]["traffic_rate_gbs"] = round(hbm, 1)
            out["roofline"]["traffic_frac_of_read_peak"] = round(
                hbm / rp["gather_pattern"], 4)
    if args.cpu_seconds > 0:
        if args.train:
            cb = cpu_baseline_train(w, dy_np, args.cpu_seconds)
            if cb is not None:
                out["cpu_baseline"] = cb
        else:
            out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
