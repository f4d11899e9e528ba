"""Paged-attention decode benchmark on one MI355X.

One step = the whole decode hot path over one batch resident in HBM: the
slot-mapped write of every sequence's new token, then decode attention over
every context. Schedules (--schedule):
  multi-query: pa_write_prefill with one query row per sequence -- the write
    and the attention in one launch of the 16x16x32-MFMA kernel, one
    workgroup per (sequence, kv head) or, with --partition, per 2048-token
    (or other) partition followed by pa_decode_splitk_reduce;
  balanced: pa_write_decode_balanced, both in one launch (work-balanced
    split-K with the log-sum-exp combine in the same kernel); with
    --separate-write, pa_write_kv_cache then pa_decode_balanced;
  partitions: pa_write_kv_cache, pa_decode over fixed partitions, then
    pa_decode_splitk_reduce;
  auto (default): the fastest measured one for the workload (AUTO_SCHEDULE).
Default workload: the largest of the five, the mixed batch with copy-on-write
shared prefixes (256 sequences, lognormal context lengths with median 1024
clipped to [16, 16384], 64 query / 8 kv heads, head_dim 128, block 32, bf16, four
groups of 64 sequences sharing a 1024-token prefix), on its default schedule;
--config 2/3/4 select the Llama-3-8B-shaped batch, the long contexts and the
int8 cache.

The KV pool is replicated R times (R x pool >= 2 GB, far above the 256 MB
last-level cache) and step i uses copy i mod R, so every step streams its KV
from HBM. Prints ONE JSON line.

value = algorithmic bytes of the step (KV in context counted once per unique
physical token, plus Q, output, block-table entries, context lengths, int8
scales, and the write's read + store of the new K/V) / step time.
W warm-up steps come first, continued until 0.1 s of steps have run (the
GPU's clocks settle over the first tens of milliseconds under load). Then two
timed passes of K steps each on the stream the kernels run on. The step
clock brackets the K steps with one pair of HIP events and nothing between
them (an event recorded between launches costs several microseconds of its
own); the kernel clock repeats the K steps with an event pair around each
launch of the decode kernel.
roofline = the decode kernel alone (with the write, when fused): its
algorithmic bytes / its mean launch duration against 8 TB/s. When the step is
that one launch, the duration is the step clock's launch period (an upper
bound that carries no marker cost); otherwise the mean of the event pairs.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

METRIC = "decode attention GB/s and % of HBM peak; seq-tokens/sec at bf16 GQA"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFS = 2500.0      # dense bf16 MFMA peak of MI355X
# smallest piece (tokens) of the balanced schedule: a few 16-token chunks per
# wave range keeps every wave of the persistent grid busy on short batches
BALANCED_MIN_PIECE = 128
WARMUP_S = 0.1
KERNEL_SOURCES = ["pa_decode_mfma.hip", "pa_decode_valu.hip", "pa_decode_common.hpp",
                  "pa_device.hpp", "pa_kernels.hpp", "pa_write_row.hpp"]


PREFILL_SOURCES = ["pa_prefill.hip", "pa_prefill.hpp", "pa_device.hpp", "pa_kernels.hpp",
                   "pa_write_row.hpp"]
# The step each workload is timed with by default: the fastest measured schedule
# (the multi-query kernel with the new tokens written in the same launch for the
# bf16 workloads, split over 4096-token partitions for the long contexts, one
# resident round of 512 workgroups: 168.6 against 170.4 us per step with 2048; the
# multi-query kernel after a separate write for the int8 batch, 118.2 against
# 124.9 us with the write fused into it and 125.0 us for the balanced kernel
# with the write fused; the balanced schedule for the mixed copy-on-write
# batch, and for the fp32 one, which the multi-query kernel does not cover).
# (schedule, partition, separate write)
AUTO_SCHEDULE = {1: ("balanced", None, False), 2: ("multi-query", 0, False),
                 3: ("multi-query", 4096, False), 4: ("multi-query", 0, True),
                 5: ("balanced", None, False)}
# The split-K partition of the long-context verify workload (4 query tokens on
# 8 x 32768 contexts): 4096 tokens, one resident round of 512 workgroups.
# Measured per step in one process: 512 tokens 203.9 us, 1024 191.1 us, 2048
# 180.1 us, 4096 170.6 us.
VERIFY_LONG_PARTITION = 4096


def source_hash(files) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "paged_kv_decode_03_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def kernel_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "paged_kv_decode_03_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(cfg: int, partition: int, schedule: str):
    """HBM bytes per decode launch from committed rocprofv3 counter runs, if
    they were taken on the current source of the kernel that runs; else None."""
    path = os.path.join(ROOT, "profiles", "decode_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    ent = rec.get(f"cfg{cfg}_P{partition}_{schedule}")
    want = (source_hash(PREFILL_SOURCES) if schedule.startswith("multi-query")
            else kernel_hash())
    if not ent or ent.get("kernel_hash") != want:
        return None
    return ent.get("bytes_per_launch")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def sample_bytes(case, seqs, np):
    """Algorithmic bytes of decoding sequences ``seqs`` alone: their unique
    physical in-context tokens' K/V, Q, output, block-table entries, lengths and
    int8 scales (the whole-batch count of synth.traffic, restricted)."""
    import synth
    B, Hkv, D = case.B, case.Hkv, case.D
    ce, ae = synth.elt_bytes(case.spec.cache), synth.elt_bytes(case.spec.act)
    slots, blocks = [], []
    for s in seqs:
        L = int(case.context_lens[s])
        p = np.arange(L)
        slots.append(case.block_tables[s, p // B].astype(np.int64) * B + p % B)
        blocks.append(case.block_tables[s, :(L + B - 1) // B])
    uniq = int(np.unique(np.concatenate(slots)).size)
    nblk = sum(len(b) for b in blocks)
    scales = (int(np.unique(np.concatenate(blocks)).size) * Hkv * 2 * 4
              if case.spec.cache == "i8" else 0)
    return uniq * 2 * Hkv * D * ce + 2 * len(seqs) * case.Hq * D * ae + 4 * nblk \
        + 4 * len(seqs) + scales


def cpu_baseline(case, budget_s: float):
    """The fp64 oracle on this host's cores, in the bench line's unit (GB/s on
    the same algorithmic byte count).

    All cores: write + decode of the whole batch, repeated until about
    ``budget_s`` seconds of work. One thread: decode of the first sequences
    (index order, about 1/8 of the batch's tokens, at least one sequence)
    repeated for about ``budget_s / 2`` seconds."""
    import numpy as np

    import oracle
    import synth
    k, v = oracle.fill_cache(case)
    tr = synth.traffic(case)
    nbytes = tr["decode"]["total"] + tr["write"]
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.write_kv_cache(case.key, case.value, k, v, case.slot_mapping, case.k_scale,
                              case.v_scale)
        oracle.decode_case(case, k, v)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 1000:
            break
    cores = oracle.num_threads()
    L = case.context_lens.astype(np.int64)
    n1 = max(1, int(np.searchsorted(np.cumsum(L), L.sum() / 8)))
    seqs = list(range(min(case.S, n1)))
    b1 = sample_bytes(case, seqs, np)
    oracle.set_num_threads(1)
    try:
        r1, t1 = 0, time.perf_counter()
        while True:
            oracle.decode_case(case, k, v, seqs=seqs)
            r1 += 1
            e1 = time.perf_counter() - t1
            if e1 >= budget_s / 2 or r1 >= 1000:
                break
    finally:
        oracle.set_num_threads(cores)
    return {"value": round(nbytes * reps / el / 1e9, 4), "unit": "GB/s", "cores": cores,
            "kind": "oracle",
            "sample": f"the whole batch (all {case.S} sequences), write + decode, "
                      f"{reps} repetitions in {el:.1f} s, fp64",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "one_thread": {"value": round(b1 * r1 / e1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                           "sample": f"decode of sequences 0..{len(seqs) - 1} "
                                     f"({int(L[seqs].sum())} context tokens), {r1} repetitions "
                                     f"in {e1:.1f} s, fp64"}}


def bench_copy_blocks(args, spec, torch, np, pa, synth):
    """pa_copy_blocks on the workload's pool: N (src, dst) pairs, sources drawn
    from the blocks in use, destinations from the free ones (or, past them, from
    a pool grown to hold them). Algorithmic bytes per pair: read + write of the
    block in both pools."""
    from gpu_helpers import fill_pool, to_device
    case = synth.make_case(spec, args.config)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    dc = to_device(case, dev)
    k, v = fill_pool(dc, dev)
    n = args.copy_blocks
    NB = case.num_blocks
    if 2 * n > NB:                                   # room for n distinct sources and destinations
        grow = 2 * n - NB
        k = torch.cat([k, torch.zeros((grow,) + tuple(k.shape[1:]), dtype=k.dtype, device=dev)])
        v = torch.cat([v, torch.zeros_like(k[NB:])])
        NB = k.shape[0]
    rng = np.random.default_rng(args.config)
    ids = rng.permutation(NB)
    mapping = torch.from_numpy(np.stack([ids[:n], ids[n:2 * n]], axis=1).astype(np.int64)).to(dev)
    ks = vs = None
    if spec.cache == "i8":
        ks = torch.ones((NB, case.Hkv), dtype=torch.float32, device=dev)
        vs = torch.ones_like(ks)
    block_bytes = case.Hkv * case.B * case.D * k.element_size()
    nbytes = n * 2 * 2 * block_bytes + n * 16 + (n * 2 * 2 * case.Hkv * 4 if ks is not None else 0)
    stream = torch.cuda.current_stream(dev)
    for _ in range(max(args.warmup, 10)):
        pa.copy_blocks(k, v, mapping, ks, vs)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        pa.copy_blocks(k, v, mapping, ks, vs)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    gbs = nbytes / (ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "copy-on-write block copy GB/s", "value": round(gbs, 2), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": spec.cache, "data": "synthetic",
        "config": {"workload": spec.name + " pool", "pairs": n, "block_bytes": block_bytes,
                   "num_kv_heads": case.Hkv, "block_size": case.B, "head_dim": case.D},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "pa_copy_blocks", "bytes_per_launch": nbytes},
    }), flush=True)


def multi_query_counts(case, qs, np):
    """Algorithmic bytes and flops of one pa_prefill launch. Bytes: K and V of
    every token of every context once per kv head (the rows of a kv head share
    its loads), the block-table entries read, Q and the output, the lengths,
    query starts and int8 scales. Flops: 4 D (p + 1) per query row and head (Q K^T
    and P V over the p + 1 tokens the row sees)."""
    L = case.context_lens.astype(np.int64)
    Hq, Hkv, D, B = case.Hq, case.Hkv, case.D, case.B
    elt = 1 if case.spec.cache == "i8" else 2
    act = 4 if case.spec.act == "f32" else 2
    nblk = (L + B - 1) // B
    kv = int(2 * Hkv * L.sum() * D * elt)
    scales = int(2 * Hkv * nblk.sum() * 4) if case.spec.cache == "i8" else 0
    T = qs.num_tokens
    nbytes = kv + scales + int(Hkv * nblk.sum() * 4) + 2 * T * Hq * D * act + 8 * case.S + 4
    seq = np.repeat(np.arange(case.S), qs.q_lens)
    pos = L[seq] - qs.q_lens[seq] + (np.arange(T) - qs.query_start_loc[seq])
    flops = int(4 * D * Hq * (pos + 1).sum())
    return nbytes, kv, flops


def bench_multi_query(args, torch, np, pa, synth):
    """pa_prefill on a multi-token workload: the speculative verify of 4 tokens
    per sequence on the Llama-shaped batch (HBM-bound: roofline against 8 TB/s)
    or 512-token prefill chunks after 3584 cached tokens (a dense contraction:
    roofline against the 2.5 PFLOP/s dense bf16 MFMA peak)."""
    from gpu_helpers import fill_pool, host_to_dev, to_device
    spec, ql = synth.MULTI_QUERY[args.multi_query]
    case = synth.make_case(spec, 2)
    qs = synth.make_queries(case, ql, 3)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    dc = to_device(case, dev)
    k0, v0 = fill_pool(dc, dev)
    pool_bytes = 2 * k0.numel() * k0.element_size()
    R = max(2, math.ceil(args.rotate_gb * 1e9 / pool_bytes))
    pools = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(R - 1)]
    q = host_to_dev(qs.q, spec.act, dev)
    qsl = torch.from_numpy(qs.query_start_loc).to(dev)
    out = torch.empty_like(q)
    mq = int(qs.q_lens.max())
    nbytes, kv, flops = multi_query_counts(case, qs, np)
    # long contexts: split-K, then the log-sum-exp reduce (--partition, else the
    # fastest measured partition size)
    P = (args.partition if args.partition is not None else VERIFY_LONG_PARTITION) \
        if args.multi_query == "verify_long" else 0
    maxL = case.max_context_len
    ws = pa.prefill_workspace(qs.num_tokens, case.Hq, case.D, maxL, P, dev) if P else None

    def step(i):
        k, v = pools[i % R]
        if P:
            pa.prefill(None, q, k, v, dc.block_tables, dc.context_lens, qsl, float(case.scale),
                       mq, maxL, dc.k_scale, dc.v_scale, partition_size=P, tmp_out=ws[0],
                       tmp_max=ws[1], tmp_sum=ws[2], row_lens=ws[3])
            pa.decode_splitk_reduce(out, ws[0], ws[1], ws[2], ws[3], maxL, P)
        else:
            pa.prefill(out, q, k, v, dc.block_tables, dc.context_lens, qsl, float(case.scale),
                       mq, maxL, dc.k_scale, dc.v_scale)

    stream = torch.cuda.current_stream(dev)
    i, t0 = 0, time.perf_counter()
    while i < args.warmup or time.perf_counter() - t0 < WARMUP_S:
        step(i)
        i += 1
        if i % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for j in range(args.steps):
        step(i + j)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    gbs = nbytes / (ms * 1e-3) / 1e9
    tfs = flops / (ms * 1e-3) / 1e12
    verify = args.multi_query.startswith("verify")
    if verify:
        roof = {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(tfs, 2), "peak": MFMA_BF16_PEAK_TFS,
                "unit": "TFLOP/s", "frac": round(tfs / MFMA_BF16_PEAK_TFS, 4)}
    traffic = None
    path = os.path.join(ROOT, "profiles", "decode_traffic.json")
    if os.path.exists(path):
        with open(path) as fh:
            ent = json.load(fh).get(f"multi_query_{args.multi_query}")
        if ent and ent.get("kernel_hash") == source_hash(PREFILL_SOURCES):
            traffic = ent["bytes_per_launch"]
    roof.update({"traffic": traffic, "kernel": "pa_prefill", "bytes_per_launch": nbytes,
                 "flops_per_launch": flops})
    line = {
        "metric": ("speculative verify attention GB/s" if verify
                   else "chunked-prefill attention TFLOP/s"),
        "value": round(gbs if verify else tfs, 2), "unit": "GB/s" if verify else "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": spec.name + (" verify, 4 query tokens per sequence" if verify
                                            else ", 512-token chunks"),
                   "partition_size": P,
                   "num_seqs": case.S, "query_tokens": qs.num_tokens,
                   "num_heads": case.Hq, "num_kv_heads": case.Hkv, "head_dim": case.D,
                   "block_size": case.B, "sum_context": int(case.context_lens.sum()),
                   "pool_copies": R},
        "gbs": round(gbs, 2), "tflops": round(tfs, 2), "roofline": roof,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = multi_query_cpu_baseline(case, qs, args.cpu_budget, verify, np)
    print(json.dumps(line), flush=True)


def multi_query_cpu_baseline(case, qs, budget_s, verify, np):
    """The fp64 oracle's ora_prefill over whole sequences (the first ones, then
    repeated) for about `budget_s` seconds, in the bench line's unit."""
    import oracle
    import synth
    k, v = oracle.fill_cache(case)
    done_b = done_f = 0
    reps, t0, s = 0, time.perf_counter(), 0
    while True:
        n = np.zeros(case.S, dtype=np.int64)
        n[s] = qs.q_lens[s]
        one = synth.Queries(query_start_loc=np.array([0] * (s + 1) + [int(n[s])] * (case.S - s),
                                                     dtype=np.int32),
                            q=qs.q[qs.query_start_loc[s]:qs.query_start_loc[s + 1]], q_lens=n)
        oracle.prefill(one.q, k, v, case.block_tables, case.context_lens, one.query_start_loc,
                       case.scale, case.k_scale, case.v_scale)
        b, _, f = multi_query_counts(case, one, np)
        done_b += b
        done_f += f
        reps += 1
        s = (s + 1) % case.S
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    val = done_b / el / 1e9 if verify else done_f / el / 1e12
    return {"value": round(val, 6), "unit": "GB/s" if verify else "TFLOP/s",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{reps} single-sequence calls of the oracle (sequences 0.., all their "
                      f"query rows) in {el:.1f} s, fp64"}


def copy_probe(torch, nbytes=1 << 30, reps=10):
    src = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    print(json.dumps({"probe": "device copy", "read_bytes": nbytes, "write_bytes": nbytes,
                      "us_per_copy": round(ms * 1e3, 2),
                      "copy_gbs": round(2 * nbytes / (ms * 1e-3) / 1e9, 1)}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=5, choices=[1, 2, 3, 4, 5],
                    help="workload (default 5: the largest, the mixed batch with copy-on-write prefixes)")
    ap.add_argument("--partition", type=int, default=None,
                    help="split-K partition (default: the workload's), or the smallest "
                         f"balanced piece in tokens (default {BALANCED_MIN_PIECE})")
    ap.add_argument("--schedule", choices=["auto", "balanced", "partitions", "multi-query"],
                    default="auto",
                    help="balanced: pa_write_decode_balanced (one launch); partitions: "
                         "pa_write_kv_cache, pa_decode, pa_decode_splitk_reduce; multi-query: "
                         "pa_write_prefill with one query row per sequence, split-K and "
                         "the reduce with --partition (with --separate-write: "
                         "pa_write_kv_cache then pa_prefill); auto (default): the fastest measured one for the "
                         "workload")
    ap.add_argument("--separate-write", action="store_true",
                    help="balanced and multi-query schedules: the write kernel, then the "
                         "decode (two launches)")
    ap.add_argument("--graph", action="store_true",
                    help="capture each step (one graph per pool copy) in a HIP graph and time "
                         "graph replays")
    ap.add_argument("--rotate-gb", type=float, default=2.0)
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-blocks", type=int, default=0, metavar="N",
                    help="instead of the decode step, time pa_copy_blocks copying N blocks of "
                         "the workload's pool (all kv heads, K and V) into free blocks")
    ap.add_argument("--multi-query", choices=["verify", "verify_long", "prefill"], default=None,
                    help="instead of the decode step, time pa_prefill: the speculative verify "
                         "of 4 tokens per sequence on the Llama-shaped batch (verify) or on the "
                         "8 x 32768 batch with split-K and the reduce (verify_long), "
                         "or 512-token prefill chunks after 3584 cached tokens (8 sequences)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only time a device copy of 1 GiB (read 1 GiB + write 1 GiB); the "
                         "reference for calibrating rocprofv3 FETCH_SIZE / WRITE_SIZE")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the paged decode path here is built and measured on a "
              "single MI355X; multi-GPU runs are not part of this build.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_probe:
        copy_probe(torch)
        return

    import paged_kv_decode_03_amd as pa
    import synth
    from gpu_helpers import fill_pool, to_device

    if args.multi_query:
        bench_multi_query(args, torch, np, pa, synth)
        return
    spec = synth.CONFIGS[args.config]
    if args.copy_blocks:
        bench_copy_blocks(args, spec, torch, np, pa, synth)
        return
    if args.schedule == "auto":
        args.schedule, auto_p, auto_sep = AUTO_SCHEDULE[args.config]
        if args.partition is None and auto_p is not None:
            args.partition = auto_p
        args.separate_write = args.separate_write or auto_sep
    balanced = args.schedule == "balanced"
    mq = args.schedule == "multi-query"
    if args.partition is not None:
        P = args.partition
    else:
        P = BALANCED_MIN_PIECE if balanced else 0 if mq else spec.partition_size
    case = synth.make_case(spec, args.config)
    tr = synth.traffic(case)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    dc = to_device(case, dev)
    k0, v0 = fill_pool(dc, dev)
    pool_bytes = 2 * k0.numel() * k0.element_size()
    R = max(2, math.ceil(args.rotate_gb * 1e9 / pool_bytes))
    pools = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(R - 1)]
    maxL = case.max_context_len
    S, Hq, D = case.S, case.Hq, case.D
    if balanced:
        ws = pa.balanced_workspace(S, Hq, case.Hkv, D, maxL, P, dev)
    elif mq:
        ws = pa.prefill_workspace(S, Hq, D, maxL, P, dev) if P > 0 else None
        qsl = torch.arange(S + 1, dtype=torch.int32, device=dev)
    else:
        ws = pa.workspace(S, Hq, D, maxL, max(P, 1), dev)
    out = torch.empty_like(dc.q)
    scale = float(case.scale)
    stream = torch.cuda.current_stream(dev)

    # the new tokens written by the decode launch itself
    fused = (balanced or mq) and not args.separate_write
    one_launch = fused and not (mq and P > 0)      # split-K adds the reduce launch

    def step(i, ev=None):
        k, v = pools[i % R]
        if fused and mq:
            if ev is not None:
                ev[0].record(stream)
            if P > 0:
                pa.write_prefill(dc.key, dc.value, dc.slot_mapping, None, dc.q, k, v,
                                 dc.block_tables, dc.context_lens, qsl, scale, 1, maxL,
                                 dc.k_scale, dc.v_scale, partition_size=P, tmp_out=ws[0],
                                 tmp_max=ws[1], tmp_sum=ws[2], row_lens=ws[3])
            else:
                pa.write_prefill(dc.key, dc.value, dc.slot_mapping, out, dc.q, k, v,
                                 dc.block_tables, dc.context_lens, qsl, scale, 1, maxL,
                                 dc.k_scale, dc.v_scale)
            if ev is not None:
                ev[1].record(stream)
            if P > 0:
                pa.decode_splitk_reduce(out, *ws[:3], ws[3], maxL, P)
            return
        if fused:
            if ev is not None:
                ev[0].record(stream)
            pa.write_decode_balanced(dc.key, dc.value, dc.slot_mapping, out, dc.q, k, v,
                                     dc.block_tables, dc.context_lens, scale, maxL, P, *ws,
                                     k_scale=dc.k_scale, v_scale=dc.v_scale)
            if ev is not None:
                ev[1].record(stream)
            return
        pa.write_kv_cache(dc.key, dc.value, k, v, dc.slot_mapping, dc.k_scale, dc.v_scale)
        if ev is not None:
            ev[0].record(stream)
        if balanced:
            pa.decode_balanced(out, dc.q, k, v, dc.block_tables, dc.context_lens, scale, maxL, P,
                               *ws, k_scale=dc.k_scale, v_scale=dc.v_scale)
        elif mq and P > 0:
            pa.prefill(None, dc.q, k, v, dc.block_tables, dc.context_lens, qsl, scale, 1, maxL,
                       dc.k_scale, dc.v_scale, partition_size=P, tmp_out=ws[0], tmp_max=ws[1],
                       tmp_sum=ws[2], row_lens=ws[3])
        elif mq:
            pa.prefill(out, dc.q, k, v, dc.block_tables, dc.context_lens, qsl, scale, 1, maxL,
                       dc.k_scale, dc.v_scale)
        elif P > 0:
            pa.decode(None, dc.q, k, v, dc.block_tables, dc.context_lens, scale, maxL, P, *ws,
                      k_scale=dc.k_scale, v_scale=dc.v_scale)
        else:
            pa.decode(out, dc.q, k, v, dc.block_tables, dc.context_lens, scale, maxL, 0,
                      k_scale=dc.k_scale, v_scale=dc.v_scale)
        if ev is not None:
            ev[1].record(stream)
        if mq and P > 0:
            pa.decode_splitk_reduce(out, *ws[:3], ws[3], maxL, P)
        elif not balanced and P > 0:
            pa.decode_splitk_reduce(out, *ws, dc.context_lens, maxL, P)

    # W warm-up steps, continued until WARMUP_S of steps have run: under load
    # the GPU's clocks take tens of milliseconds to settle.
    w0, t0 = 0, time.perf_counter()
    while w0 < args.warmup or time.perf_counter() - t0 < WARMUP_S:
        step(w0)
        w0 += 1
        if w0 % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    run = step
    if args.graph:
        # one graph per pool copy, captured on a side stream (the step's kernels
        # allocate nothing and clear nothing with memsets, so they capture as is)
        graphs = []
        cap = torch.cuda.Stream(dev)
        cap.wait_stream(stream)
        for r in range(R):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                step(r)
            graphs.append(g)
        torch.cuda.synchronize()

        def run(i, ev=None):
            if ev is not None:
                ev[0].record(stream)
            graphs[i % R].replay()
            if ev is not None:
                ev[1].record(stream)
        for i in range(2 * R):
            run(i)
        torch.cuda.synchronize()
    # 1. the step clock: K steps with nothing recorded between the two events
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record(stream)
    for i in range(args.steps):
        run(w0 + i)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t_start.elapsed_time(t_end) / args.steps
    # 2. the kernel clock: the same K steps again, with an event pair around
    # each launch of the decode kernel
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for i in range(args.steps):
        run(w0 + args.steps + i, evs[i])
    torch.cuda.synchronize()
    pair_ms = np.array([a.elapsed_time(b) for a, b in evs])
    # One launch per step: the launch period of pass 1 bounds the launch's
    # duration from above, and unlike an event pair it carries no marker cost.
    # with graphs the event pairs wrap a whole replay, so the step clock is used
    dec_mean = ms_per_step if one_launch or args.graph else float(pair_ms.mean())

    step_bytes = tr["decode"]["total"] + tr["write"]
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    # the timed unit: the decode launch, or with graphs the whole step's replay
    kernel_bytes = tr["decode"]["total"] + (tr["write"] if fused or args.graph else 0)
    achieved = kernel_bytes / (dec_mean * 1e-3) / 1e9
    sched = ("fused" if balanced else "multi-query-fused") if fused else args.schedule
    traffic = measured_traffic(args.config, P, sched)
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": w0,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "bf16": "bf16"}[spec.act] + ("+i8kv" if spec.cache == "i8" else ""),
        "data": "synthetic",
        "config": {
            "workload": spec.name, "cfg": args.config, "num_seqs": S, "num_heads": Hq,
            "num_kv_heads": case.Hkv, "head_dim": D, "block_size": case.B,
            "context_lens": list(spec.lens), "sum_context": tr["sum_len"],
            "unique_kv_tokens": tr["unique_tokens"], "partition_size": P, "pool_copies": R,
            "schedule": args.schedule + ("" if fused or not (balanced or mq) else " (separate write)")
                        + (", HIP graph replays" if args.graph else ""),
            "step": ("write + balanced split-K decode + combine, one launch" if fused and balanced
                     else "write + multi-query kernel with one row per sequence, one launch" +
                     ("; reduce" if P else "") if fused else
                     "write; balanced split-K decode (combine fused)" if balanced else
                     "write; multi-query kernel with one row per sequence" +
                     ("; reduce" if P else "") if mq else
                     "write; split-K decode; reduce" if P else "write; one-pass decode"),
        },
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "seq_tokens_per_s": round(S / (ms_per_step * 1e-3), 1),
        "context_tokens_per_s": round(tr["sum_len"] / (ms_per_step * 1e-3), 1),
        "decode_kernel_us": {"mean": round(dec_mean * 1e3, 2),
                             "clock": ("launch period" if one_launch or args.graph
                                       else "event pairs"),
                             "event_pairs": {
                                 "mean": round(float(pair_ms.mean()) * 1e3, 2),
                                 "p10": round(float(np.percentile(pair_ms, 10)) * 1e3, 2),
                                 "p90": round(float(np.percentile(pair_ms, 90)) * 1e3, 2)}},
        "bytes": {"decode": tr["decode"]["total"], "kv": tr["decode"]["kv"],
                  "kv_logical": tr["decode"]["kv_logical"], "write": tr["write"]},
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": ("graph replay of the whole step" if args.graph and not fused else
                       "pa_write_decode_balanced" if fused and balanced else
                       "pa_write_prefill" + (" (split-K partials)" if P else "") if fused else
                       "pa_decode_balanced" if balanced else
                       "pa_prefill" + (" (split-K partials)" if P else "") if mq else
                       "pa_decode (split-K partials)" if P else "pa_decode"),
            "bytes_per_launch": kernel_bytes,
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        del pools
        torch.cuda.empty_cache()
        res["cpu_baseline"] = cpu_baseline(case, args.cpu_budget)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
