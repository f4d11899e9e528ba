"""The decode step captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

Every entry point enqueues only kernels (no allocation, no memset: the
balanced schedule's counters are reset by the kernel itself), so a step can be
captured once and replayed: the fused balanced step (with a caller workspace,
or without one), write + split-K decode + reduce, and the default step on bf16
batches (the write fused with the multi-query kernel, one pass or split with
the reduce). Each test replays the graph several times, with
eager launches of the same entry points and synchronisations in between, and
checks every replay bit for bit against the eager result of the same step
(the schedules are static, so eager and replayed results are the same bits),
and the written pool byte for byte against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import as_f64, dev_to_host, poison_pool, to_device, tol

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import paged_kv_decode_03_amd as pa

C = synth.CONFIGS
SPECS = {
    "cfg2s": C[2].replace(num_seqs=12, lens=("uniform", 1, 1100), max_len=1100),
    "cfg4s": C[4].replace(num_seqs=10, lens=("uniform", 1, 1300), max_len=1300),
    "cfg5s": C[5].replace(num_seqs=16, lens=("lognormal", 200, 1.0, 1, 1500), max_len=1500,
                          prefix_groups=2, prefix_tokens=256),
    "cfg3s": C[3].replace(num_seqs=2, lens=("const", 4099), max_len=4099),
}


def pre_pool(case, dc):
    k, v = poison_pool(case)
    if dc.pre_slots.numel():
        pa.write_kv_cache(dc.pre_key, dc.pre_value, k, v, dc.pre_slots, dc.k_scale, dc.v_scale)
    return k, v


def make_step(case, dc, k, v, out, schedule):
    maxL, scale = case.max_context_len, float(case.scale)
    if schedule == "fused":
        ws = pa.balanced_workspace(case.S, case.Hq, case.Hkv, case.D, maxL, 64, "cuda")

        def step():
            pa.write_decode_balanced(dc.key, dc.value, dc.slot_mapping, out, dc.q, k, v,
                                     dc.block_tables, dc.context_lens, scale, maxL, 64, *ws,
                                     k_scale=dc.k_scale, v_scale=dc.v_scale)
        return step, ws
    if schedule == "noalloc":
        def step():
            pa.write_decode_balanced_noalloc(dc.key, dc.value, dc.slot_mapping, out, dc.q, k, v,
                                             dc.block_tables, dc.context_lens, scale, maxL, 64,
                                             k_scale=dc.k_scale, v_scale=dc.v_scale)
        return step, None
    if schedule.startswith("multi-query"):
        # the default step on bf16 batches: pa_write_prefill with one query row
        # per sequence, in one pass or split over P-token partitions + the reduce;
        # "multi-query-sep" (the int8 batch's default): pa_write_kv_cache, then
        # pa_prefill
        P = int(schedule.split(":")[1]) if ":" in schedule else 0
        sep = schedule.startswith("multi-query-sep")
        qsl = torch.arange(case.S + 1, dtype=torch.int32, device="cuda")
        ws = pa.prefill_workspace(case.S, case.Hq, case.D, maxL, P, "cuda") if P else None
        ks, vs = dc.k_scale, dc.v_scale

        def step():
            if sep:
                pa.write_kv_cache(dc.key, dc.value, k, v, dc.slot_mapping, ks, vs)
                pa.prefill(out, dc.q, k, v, dc.block_tables, dc.context_lens, qsl, scale, 1,
                           maxL, ks, vs)
            elif P:
                pa.write_prefill(dc.key, dc.value, dc.slot_mapping, None, dc.q, k, v,
                                 dc.block_tables, dc.context_lens, qsl, scale, 1, maxL, ks, vs,
                                 partition_size=P, tmp_out=ws[0], tmp_max=ws[1], tmp_sum=ws[2],
                                 row_lens=ws[3])
                pa.decode_splitk_reduce(out, *ws[:3], ws[3], maxL, P)
            else:
                pa.write_prefill(dc.key, dc.value, dc.slot_mapping, out, dc.q, k, v,
                                 dc.block_tables, dc.context_lens, qsl, scale, 1, maxL, ks, vs)
        return step, ws
    P = case.spec.partition_size or 512
    ws = pa.workspace(case.S, case.Hq, case.D, maxL, P, "cuda")

    def step():
        pa.write_kv_cache(dc.key, dc.value, k, v, dc.slot_mapping, dc.k_scale, dc.v_scale)
        pa.decode(None, dc.q, k, v, dc.block_tables, dc.context_lens, scale, maxL, P, *ws,
                  k_scale=dc.k_scale, v_scale=dc.v_scale)
        pa.decode_splitk_reduce(out, *ws, dc.context_lens, maxL, P)
    return step, ws


@pytest.mark.parametrize("name,schedule", [("cfg2s", "fused"), ("cfg4s", "fused"),
                                           ("cfg5s", "fused"), ("cfg3s", "partitions"),
                                           ("cfg2s", "partitions"), ("cfg2s", "multi-query"),
                                           ("cfg3s", "multi-query:2048"), ("cfg5s", "noalloc"),
                                           ("cfg4s", "noalloc"), ("cfg4s", "multi-query-sep"),
                                           ("cfg4s", "multi-query")])
def test_graph_replays_match_eager(name, schedule):
    print(f"[graph] {name} {schedule}", flush=True)
    case = synth.make_case(SPECS[name], 21)
    dc = to_device(case)
    ok, ov = oracle.fill_cache(case)
    ref = oracle.decode_case(case, ok, ov)
    # eager: the step on its own pool
    ke, ve = pre_pool(case, dc)
    out_e = torch.full_like(dc.q, float("nan"))
    step_e, _ = make_step(case, dc, ke, ve, out_e, schedule)
    step_e()
    torch.cuda.synchronize()
    want = dev_to_host(out_e)
    assert np.array_equal(dev_to_host(ke).view(np.uint8), ok.view(np.uint8))
    assert np.abs(as_f64(out_e) - ref).max() <= tol(case)
    # captured: the same step on a second pool; warm up once outside the capture
    kg, vg = pre_pool(case, dc)
    out_g = torch.full_like(dc.q, float("nan"))
    step_g, ws = make_step(case, dc, kg, vg, out_g, schedule)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        step_g()
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step_g()
    torch.cuda.synchronize()
    for rep in range(4):
        out_g.fill_(float("nan"))
        g.replay()
        step_e()                                     # eager work between replays
        torch.cuda.synchronize()
        assert np.array_equal(dev_to_host(out_g), want), f"replay {rep} differs from eager"
        assert np.array_equal(dev_to_host(out_e), want), f"eager after replay {rep} differs"
    assert np.array_equal(dev_to_host(kg).view(np.uint8), ok.view(np.uint8)), "k pool"
    assert np.array_equal(dev_to_host(vg).view(np.uint8), ov.view(np.uint8)), "v pool"
    if schedule == "fused":
        assert int(ws[3].abs().sum()) == 0, "counters not reset"
