"""pa_prefill (several new query tokens per sequence: speculative verify and
chunked prefill) against the fp64 oracle, through the C ABI.

Small batches are compared element by element with ``oracle.prefill``. The
full-size workloads compare sampled rows with one-token decode over the
context cut after the row's position, which the oracle's own pins tie to
``oracle.prefill`` row by row. Tolerances are those of the decode path
(bf16 2e-2, int8 3e-2 max abs)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import as_f64, fill_pool, host_to_dev, run_decode, to_device, tol

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import paged_kv_decode_03_amd as pa

S_ = synth.Spec
CASES = {
    # name: (spec, query counts)
    "verify_g4": (synth.CONFIGS[2].replace(num_seqs=12, lens=("uniform", 1, 1100), max_len=1100),
                  ("const", 4)),
    "verify_g4_i8": (synth.CONFIGS[4].replace(num_seqs=10, lens=("uniform", 1, 1300),
                                              max_len=1300), ("const", 4)),
    "verify_g8_b32": (S_("G=8 B=32", 8, ("uniform", 1, 900), 32, 4, 128, 32, act="bf16",
                         cache="bf16", max_len=900), ("uniform", 1, 8)),
    "g2_i8_b32": (S_("G=2 int8 B=32", 6, ("uniform", 1, 700), 8, 4, 128, 32, act="bf16",
                     cache="i8", max_len=700), ("uniform", 0, 20)),
    "g16": (S_("G=16", 5, ("uniform", 1, 600), 16, 1, 128, 16, act="bf16", cache="bf16",
               max_len=600), ("uniform", 1, 3)),
    "mixed_g4": (S_("G=4 mixed counts", 9, ("uniform", 1, 800), 16, 4, 128, 16, act="bf16",
                    cache="bf16", max_len=800), ("uniform", 0, 40)),
    "chunk_g4": (S_("G=4 prefill chunk", 2, ("const", 1500), 8, 2, 128, 16, act="bf16",
                    cache="bf16", max_len=1500), ("const", 300)),
    "chunk_i8_g8": (S_("G=8 int8 prefill chunk", 2, ("uniform", 600, 1000), 16, 2, 128, 32,
                       act="bf16", cache="i8", max_len=1000), ("const", 100)),
    "whole_mha": (S_("MHA whole-context prefill", 3, ("uniform", 1, 200), 4, 4, 128, 16,
                     act="bf16", cache="bf16", max_len=200), "whole"),
    "cow_g8": (synth.CONFIGS[5].replace(num_seqs=16, lens=("lognormal", 200, 1.0, 1, 1500),
                                        max_len=1500, prefix_groups=2, prefix_tokens=256),
               ("uniform", 1, 5)),
    # one row per sequence, no split: up to 256 sequences (a multiple of 8) are
    # placed on the XCDs by context length; many equal lengths at 64, the
    # largest batch placed so at 256, the plain order at 264
    "decode_ties_s64": (synth.CONFIGS[2].replace(num_seqs=64, lens=("uniform", 1, 40),
                                                 max_len=40), ("const", 1)),
    "decode_s256": (synth.CONFIGS[2].replace(num_seqs=256, lens=("uniform", 1, 300),
                                             max_len=300), ("const", 1)),
    "decode_s264": (synth.CONFIGS[2].replace(num_seqs=264, lens=("uniform", 1, 300),
                                             max_len=300), ("const", 1)),
}


def prepare(name, seed=11):
    spec, ql = CASES[name]
    case = synth.make_case(spec, seed)
    if ql == "whole":
        ql = case.context_lens.astype(np.int64)
    qs = synth.make_queries(case, ql, seed + 1)
    dc = to_device(case)
    fill_pool(dc)
    return case, qs, dc


def run_prefill(case, qs, dc, max_query_len=None, partition_size=0):
    """pa_prefill in one pass, or split-K partials then pa_decode_splitk_reduce."""
    q = host_to_dev(qs.q, case.spec.act, "cuda")
    qsl = torch.from_numpy(qs.query_start_loc).cuda()
    out = torch.full_like(q, float("nan"))
    mq = int(qs.q_lens.max()) if max_query_len is None else max_query_len
    maxL = case.max_context_len
    if partition_size:
        ws = pa.prefill_workspace(qs.num_tokens, case.Hq, case.D, maxL, partition_size, "cuda")
        for t in ws[:3]:
            t.fill_(float("nan"))
        pa.prefill(None, q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens, qsl,
                   float(case.scale), mq, maxL, dc.k_scale, dc.v_scale,
                   partition_size=partition_size, tmp_out=ws[0], tmp_max=ws[1], tmp_sum=ws[2],
                   row_lens=ws[3])
        pa.decode_splitk_reduce(out, ws[0], ws[1], ws[2], ws[3], maxL, partition_size)
    else:
        pa.prefill(out, q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens, qsl,
                   float(case.scale), mq, maxL, dc.k_scale, dc.v_scale)
    torch.cuda.synchronize()
    return as_f64(out)


@pytest.mark.parametrize("name", list(CASES))
def test_prefill_parity(name):
    case, qs, dc = prepare(name)
    print(f"[prefill] {name}: {qs.num_tokens} query rows, max {int(qs.q_lens.max())} per seq",
          flush=True)
    got = run_prefill(case, qs, dc)
    ok, ov = oracle.fill_cache(case)
    ref = oracle.prefill(qs.q, ok, ov, case.block_tables, case.context_lens, qs.query_start_loc,
                         case.scale, case.k_scale, case.v_scale)
    assert np.isfinite(got).all()
    err = np.abs(got - ref).max()
    print(f"[prefill] {name}: max |gpu - oracle| = {err:.3e}", flush=True)
    assert err <= tol(case), f"{name}: max |gpu - oracle| = {err}"


@pytest.mark.parametrize("name,P", [("verify_g4", 64), ("verify_g4_i8", 512),
                                    ("verify_g8_b32", 32), ("g2_i8_b32", 96),
                                    ("mixed_g4", 128), ("chunk_g4", 256), ("whole_mha", 32),
                                    ("cow_g8", 512)])
def test_prefill_splitk_parity(name, P):
    """Split-K over each row's tokens, combined by the decode reduce with the
    rows' own lengths, against the oracle; also the row lengths themselves."""
    case, qs, dc = prepare(name)
    got = run_prefill(case, qs, dc, partition_size=P)
    ok, ov = oracle.fill_cache(case)
    ref = oracle.prefill(qs.q, ok, ov, case.block_tables, case.context_lens, qs.query_start_loc,
                         case.scale, case.k_scale, case.v_scale)
    assert np.isfinite(got).all()
    err = np.abs(got - ref).max()
    print(f"[prefill split-K] {name} P={P}: max |gpu - oracle| = {err:.3e}", flush=True)
    assert err <= tol(case), f"{name} P={P}: max |gpu - oracle| = {err}"


def test_prefill_splitk_row_lens():
    case, qs, dc = prepare("mixed_g4")
    q = host_to_dev(qs.q, case.spec.act, "cuda")
    qsl = torch.from_numpy(qs.query_start_loc).cuda()
    ws = pa.prefill_workspace(qs.num_tokens, case.Hq, case.D, case.max_context_len, 64, "cuda")
    ws[3].fill_(-1)
    pa.prefill(None, q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens, qsl,
               float(case.scale), int(qs.q_lens.max()), case.max_context_len,
               partition_size=64, tmp_out=ws[0], tmp_max=ws[1], tmp_sum=ws[2], row_lens=ws[3])
    seq = np.repeat(np.arange(case.S), qs.q_lens)
    pos = case.context_lens[seq] - qs.q_lens[seq] + (np.arange(qs.num_tokens)
                                                      - qs.query_start_loc[seq])
    assert np.array_equal(ws[3].cpu().numpy(), (pos + 1).astype(np.int32))


def test_prefill_one_token_matches_decode():
    """n_s = 1 is decode: the same rows as the decode kernels, to tolerance."""
    spec = synth.CONFIGS[2].replace(num_seqs=8, lens=("uniform", 1, 700), max_len=700)
    case = synth.make_case(spec, 5)
    dc = to_device(case)
    fill_pool(dc)
    qs = synth.Queries(query_start_loc=np.arange(case.S + 1, dtype=np.int32), q=case.q,
                       q_lens=np.ones(case.S, dtype=np.int64))
    got = run_prefill(case, qs, dc)
    dec = as_f64(run_decode(dc, 0))
    assert np.abs(got - dec).max() <= tol(case)


def test_prefill_loose_max_query_len():
    """A max_query_len above every count launches more row tiles; the extra
    tiles find no rows and the result is the same."""
    case, qs, dc = prepare("mixed_g4")
    a = run_prefill(case, qs, dc)
    b = run_prefill(case, qs, dc, max_query_len=case.max_context_len)
    assert np.array_equal(a, b)


def test_prefill_no_rows():
    """Sequences with no new tokens, and a batch with none at all."""
    case, qs, dc = prepare("verify_g4")
    n = qs.q_lens.copy()
    n[::2] = 0
    qz = synth.make_queries(case, n, 3)
    got = run_prefill(case, qz, dc)
    ok, ov = oracle.fill_cache(case)
    ref = oracle.prefill(qz.q, ok, ov, case.block_tables, case.context_lens,
                         qz.query_start_loc, case.scale)
    assert np.abs(got - ref).max() <= tol(case)
    empty = synth.make_queries(case, np.zeros(case.S, dtype=np.int64), 3)
    assert run_prefill(case, empty, dc, max_query_len=0).size == 0


@pytest.mark.timeout(600)
@pytest.mark.parametrize("cfg,P,sep", [(2, 0, False), (3, 4096, False), (4, 0, True),
                                       (4, 0, False)])
def test_default_step_full_size_sampled(cfg, P, sep):
    """The default decode step of the Llama-shaped batch (one pass), of the
    long contexts (4096-token partitions, then the reduce) and of the int8
    batch at full size, in the launch configuration the bench times:
    pa_write_prefill with one query row per sequence writes the new tokens
    (their slots hold poison before) and attends; on the int8 batch
    pa_write_kv_cache then pa_prefill (sep), and the fused int8 write too. The
    pool is byte-identical to the oracle's; sampled sequences (every head and
    dim) are checked against the oracle's decode."""
    from gpu_helpers import poison_pool
    spec = synth.CONFIGS[cfg]
    print(f"[default step] cfg{cfg} P={P}: generating", flush=True)
    case = synth.make_case(spec, cfg)
    dc = to_device(case)
    k, v = poison_pool(case)
    if dc.pre_slots.numel():
        pa.write_kv_cache(dc.pre_key, dc.pre_value, k, v, dc.pre_slots, dc.k_scale, dc.v_scale)
    qsl = torch.arange(case.S + 1, dtype=torch.int32, device="cuda")
    out = torch.full_like(dc.q, float("nan"))
    maxL = case.max_context_len
    print(f"[default step] cfg{cfg} P={P} separate write {sep}: gpu", flush=True)
    if sep:
        pa.write_kv_cache(dc.key, dc.value, k, v, dc.slot_mapping, dc.k_scale, dc.v_scale)
        pa.prefill(out, dc.q, k, v, dc.block_tables, dc.context_lens, qsl, float(case.scale), 1,
                   maxL, dc.k_scale, dc.v_scale)
    elif P:
        ws = pa.prefill_workspace(case.S, case.Hq, case.D, maxL, P, "cuda")
        pa.write_prefill(dc.key, dc.value, dc.slot_mapping, None, dc.q, k, v, dc.block_tables,
                         dc.context_lens, qsl, float(case.scale), 1, maxL, dc.k_scale,
                         dc.v_scale, partition_size=P, tmp_out=ws[0], tmp_max=ws[1],
                         tmp_sum=ws[2], row_lens=ws[3])
        pa.decode_splitk_reduce(out, ws[0], ws[1], ws[2], ws[3], maxL, P)
    else:
        pa.write_prefill(dc.key, dc.value, dc.slot_mapping, out, dc.q, k, v, dc.block_tables,
                         dc.context_lens, qsl, float(case.scale), 1, maxL, dc.k_scale,
                         dc.v_scale)
    torch.cuda.synchronize()
    got = as_f64(out)
    assert np.isfinite(got).all()
    from gpu_helpers import dev_to_host
    ok, ov = oracle.fill_cache(case)
    assert np.array_equal(dev_to_host(k).view(np.uint8), ok.view(np.uint8)), "K pool differs"
    assert np.array_equal(dev_to_host(v).view(np.uint8), ov.view(np.uint8)), "V pool differs"
    L = case.context_lens
    rng = np.random.default_rng(cfg)
    seqs = sorted({int(np.argmax(L)), int(np.argmin(L)), 0, case.S - 1,
                   *[int(x) for x in rng.choice(case.S, size=2, replace=False)]})
    if cfg == 3:
        seqs = seqs[:2]
    print(f"[default step] cfg{cfg} P={P}: oracle on sequences {seqs}", flush=True)
    ref = oracle.decode_case(case, ok, ov, seqs=seqs)
    err = np.abs(got[seqs] - ref).max()
    print(f"[default step] cfg{cfg} P={P}: max err {err:.3e}", flush=True)
    assert err <= tol(case)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,P", [("verify", 0), ("prefill", 0), ("verify_long", 512),
                                    ("verify_long", 4096)])
def test_prefill_full_size_sampled(name, P):
    """(verify_long at 4096-token partitions is the launch bench.py times.)"""
    spec, ql = synth.MULTI_QUERY[name]
    print(f"[prefill full] {name}: generating", flush=True)
    case = synth.make_case(spec, 2)
    qs = synth.make_queries(case, ql, 3)
    dc = to_device(case)
    fill_pool(dc)
    print(f"[prefill full] {name}: gpu, {qs.num_tokens} rows", flush=True)
    got = run_prefill(case, qs, dc, partition_size=P)
    assert np.isfinite(got).all()
    rng = np.random.default_rng(4)
    rows = np.unique(np.concatenate([rng.choice(qs.num_tokens, size=24, replace=False),
                                     qs.query_start_loc[1:] - 1, [0]]))
    seq = np.searchsorted(qs.query_start_loc, rows, side="right") - 1
    pos = case.context_lens[seq] - qs.q_lens[seq] + (rows - qs.query_start_loc[seq])
    ok, ov = oracle.fill_cache(case)
    print(f"[prefill full] {name}: oracle on {len(rows)} rows", flush=True)
    ref = oracle.decode(qs.q[rows], ok, ov, case.block_tables[seq], (pos + 1).astype(np.int32),
                        case.scale, case.k_scale, case.v_scale)
    err = np.abs(got[rows] - ref).max()
    print(f"[prefill full] {name}: max err {err:.3e}", flush=True)
    assert err <= tol(case)


# ---- pa_write_prefill: the new tokens written by the same launch ------------

def new_token_rows(case, qs):
    """key / value rows [T, Hkv, D] and slots [T] of every sequence's n_s newest
    tokens (the query rows), taken from the batch's source draws."""
    import pins
    idx, kall, vall = pins.source_rows(case)
    seq = np.repeat(np.arange(case.S), qs.q_lens)
    pos = case.context_lens[seq] - qs.q_lens[seq] + (np.arange(qs.num_tokens)
                                                      - qs.query_start_loc[seq])
    slots = case.block_tables[seq, pos // case.B].astype(np.int64) * case.B + pos % case.B
    rows = idx[slots]
    assert (rows >= 0).all()
    return kall[rows], vall[rows], slots


# (the copy-on-write batch takes one new token per sequence: a new token is
# never in a shared prefix block there, as in a real copy-on-write pool)
@pytest.mark.parametrize("name,P", [("verify_g4", 0), ("verify_g8_b32", 0), ("mixed_g4", 0),
                                    ("chunk_g4", 0), ("whole_mha", 0), ("cow_g8", 0),
                                    ("decode_ties_s64", 0), ("decode_s256", 0),
                                    ("verify_g4", 64), ("chunk_g4", 256), ("cow_g8", 512),
                                    ("verify_g4_i8", 0), ("g2_i8_b32", 0), ("chunk_i8_g8", 0),
                                    ("verify_g4_i8", 64), ("chunk_i8_g8", 256)])
def test_write_prefill_parity(name, P):
    """One launch writes the new tokens and attends: the pool afterwards is
    byte-identical to the oracle's write (int8: the oracle's codes under the
    block scales), the output within tolerance of the oracle. The new tokens'
    slots hold poison (NaN, int8 -128) before the call."""
    spec, ql = CASES[name]
    if name == "cow_g8":
        ql = ("const", 1)
    case = synth.make_case(spec, 11)
    if ql == "whole":
        ql = case.context_lens.astype(np.int64)
    qs = synth.make_queries(case, ql, 12)
    ok, ov = oracle.fill_cache(case)
    kn, vn, slots = new_token_rows(case, qs)
    kp, vp = ok.copy(), ov.copy()
    flat_k = kp.reshape(case.num_blocks, case.Hkv, case.B, case.D)
    flat_v = vp.reshape(case.num_blocks, case.Hkv, case.B, case.D)
    poison = synth.I8_POISON if case.spec.cache == "i8" else synth.BF16_POISON
    flat_k[slots // case.B, :, slots % case.B, :] = poison
    flat_v[slots // case.B, :, slots % case.B, :] = poison
    k = host_to_dev(kp, case.spec.cache, "cuda")
    v = host_to_dev(vp, case.spec.cache, "cuda")
    dc = to_device(case)
    q = host_to_dev(qs.q, "bf16", "cuda")
    qsl = torch.from_numpy(qs.query_start_loc).cuda()
    out = torch.full_like(q, float("nan"))
    maxL = case.max_context_len
    args = (host_to_dev(kn, "bf16", "cuda"), host_to_dev(vn, "bf16", "cuda"),
            torch.from_numpy(slots).cuda())
    if P:
        ws = pa.prefill_workspace(qs.num_tokens, case.Hq, case.D, maxL, P, "cuda")
        pa.write_prefill(*args, None, q, k, v, dc.block_tables, dc.context_lens, qsl,
                         float(case.scale), int(qs.q_lens.max()), maxL, dc.k_scale, dc.v_scale,
                         partition_size=P, tmp_out=ws[0], tmp_max=ws[1], tmp_sum=ws[2],
                         row_lens=ws[3])
        pa.decode_splitk_reduce(out, ws[0], ws[1], ws[2], ws[3], maxL, P)
    else:
        pa.write_prefill(*args, out, q, k, v, dc.block_tables, dc.context_lens, qsl,
                         float(case.scale), int(qs.q_lens.max()), maxL, dc.k_scale, dc.v_scale)
    torch.cuda.synchronize()
    from gpu_helpers import dev_to_host
    assert np.array_equal(dev_to_host(k).view(np.uint8), ok.view(np.uint8)), "K pool differs"
    assert np.array_equal(dev_to_host(v).view(np.uint8), ov.view(np.uint8)), "V pool differs"
    got = as_f64(out)
    ref = oracle.prefill(qs.q, ok, ov, case.block_tables, case.context_lens, qs.query_start_loc,
                         case.scale, case.k_scale, case.v_scale)
    assert np.isfinite(got).all()
    err = np.abs(got - ref).max()
    print(f"[write_prefill] {name} P={P}: max |gpu - oracle| = {err:.3e}", flush=True)
    assert err <= tol(case)


@pytest.mark.parametrize("name", ["verify_g4", "verify_g4_i8", "g2_i8_b32", "chunk_i8_g8"])
def test_write_prefill_matches_two_calls(name):
    """Bit-identical to pa_write_kv_cache followed by pa_prefill (output and
    pool)."""
    case, qs, dc = prepare(name)
    kn, vn, slots = new_token_rows(case, qs)
    args = (host_to_dev(kn, "bf16", "cuda"), host_to_dev(vn, "bf16", "cuda"),
            torch.from_numpy(slots).cuda())
    q = host_to_dev(qs.q, "bf16", "cuda")
    qsl = torch.from_numpy(qs.query_start_loc).cuda()
    k2, v2 = dc.k_cache.clone(), dc.v_cache.clone()
    a = torch.empty_like(q)
    b = torch.empty_like(q)
    mq, maxL = int(qs.q_lens.max()), case.max_context_len
    ks, vs = dc.k_scale, dc.v_scale
    pa.write_prefill(*args, a, q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens, qsl,
                     float(case.scale), mq, maxL, ks, vs)
    pa.write_kv_cache(args[0], args[1], k2, v2, args[2], ks, vs)
    pa.prefill(b, q, k2, v2, dc.block_tables, dc.context_lens, qsl, float(case.scale), mq, maxL,
               ks, vs)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    iv = torch.int8 if case.spec.cache == "i8" else torch.int16    # bits (the pool holds NaN)
    assert torch.equal(dc.k_cache.view(iv), k2.view(iv))
    assert torch.equal(dc.v_cache.view(iv), v2.view(iv))


def test_pa_check_rejects_bad_queries(monkeypatch):
    """PA_CHECK=1 validates the query layout and the new tokens' slots on the
    host (nothing is launched): starts that do not end at the row count, more
    rows than context, more rows than max_query_len, a slot that is not its
    token's position."""
    case, qs, dc = prepare("verify_g4")
    q = host_to_dev(qs.q, "bf16", "cuda")
    out = torch.empty_like(q)
    maxL = case.max_context_len
    monkeypatch.setenv("PA_CHECK", "1")

    def call(qsl_np, mq):
        qsl = torch.from_numpy(qsl_np.astype(np.int32)).cuda()
        pa.prefill(out, q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens, qsl,
                   float(case.scale), mq, maxL)

    good = qs.query_start_loc.copy()
    call(good, 4)                                   # accepted
    bad = good.copy()
    bad[-1] -= 1                                    # does not end at num_query_tokens
    with pytest.raises(pa.PAError) as e:
        call(bad, 4)
    assert e.value.status == -7
    with pytest.raises(pa.PAError) as e:
        call(good, 3)                               # a sequence has more rows than max_query_len
    assert e.value.status == -7
    lens = dc.context_lens.clone()
    lens[0] = 2                                     # fewer tokens than its 4 rows
    with pytest.raises(pa.PAError) as e:
        pa.prefill(out, q, dc.k_cache, dc.v_cache, dc.block_tables, lens,
                   torch.from_numpy(good).cuda(), float(case.scale), 4, maxL)
    assert e.value.status == -7
    kn, vn, slots = new_token_rows(case, qs)
    bad_slots = slots.copy()
    bad_slots[0] += 1                               # not the slot of its position
    with pytest.raises(pa.PAError) as e:
        pa.write_prefill(host_to_dev(kn, "bf16", "cuda"), host_to_dev(vn, "bf16", "cuda"),
                         torch.from_numpy(bad_slots).cuda(), out, q, dc.k_cache.clone(),
                         dc.v_cache.clone(), dc.block_tables, dc.context_lens,
                         torch.from_numpy(good).cuda(), float(case.scale), 4, maxL)
    assert e.value.status == -7


# ---- exactness: one-hot probes, L = 1, placement, negative slots ------------

EXACT = {
    # name: (spec, query rows per sequence); rows <= 16 per (seq, kv head): one
    # row block (the decode and verify shape); more: two row blocks, 64-row
    # and 128-row tiles
    "g4_b16": (synth.CONFIGS[2].replace(num_seqs=12, lens=("uniform", 1, 900), max_len=900), 1),
    "g4_b16_rows4": (synth.CONFIGS[2].replace(num_seqs=12, lens=("uniform", 1, 900),
                                              max_len=900), 4),
    "g8_b32_cow": (synth.CONFIGS[5].replace(num_seqs=16, lens=("lognormal", 200, 1.0, 1, 1500),
                                            max_len=1500, prefix_groups=2, prefix_tokens=256), 1),
    "g8_b32_cow_rows3": (synth.CONFIGS[5].replace(num_seqs=16,
                                                  lens=("lognormal", 200, 1.0, 1, 1500),
                                                  max_len=1500, prefix_groups=2,
                                                  prefix_tokens=256), 3),
    "g4_i8_b16": (synth.CONFIGS[4].replace(num_seqs=10, lens=("uniform", 1, 1300),
                                           max_len=1300), 1),
    "g4_i8_b16_rows4": (synth.CONFIGS[4].replace(num_seqs=10, lens=("uniform", 1, 1300),
                                                 max_len=1300), 4),
    "g2_i8_b32_rows6": (S_("G=2 int8 B=32", 6, ("uniform", 1, 700), 8, 4, 128, 32, act="bf16",
                           cache="i8", max_len=700), 6),
    "g1_rows20": (S_("MHA 20 rows", 4, ("uniform", 1, 500), 4, 4, 128, 16, act="bf16",
                     cache="bf16", max_len=500), 20),
    "g4_rows40": (S_("G=4 40 rows", 3, ("uniform", 40, 700), 8, 2, 128, 16, act="bf16",
                     cache="bf16", max_len=700), 40),
    "g8_i8_rows100": (S_("G=8 int8 100 rows", 2, ("uniform", 100, 600), 16, 2, 128, 32,
                         act="bf16", cache="i8", max_len=600), 100),
}


def _onehot_prefill(name, seed, rng):
    """One-hot batch with query rows: every row of sequence s (positions L - n ..
    L - 1) sees its probe t* <= L - n, which lies in a block s owns alone. A
    sequence whose private blocks start after L - rows takes fewer rows."""
    from probe_cases import onehot_case, onehot_queries
    spec, rows = EXACT[name]
    base = synth.make_case(spec, seed)
    L0 = base.context_lens.astype(np.int64)
    n = np.minimum(rows, L0)
    for s in range(base.S):
        first_own = next(t for t in range(int(L0[s]))
                         if base.refcount[base.block_tables[s, t // base.B]] == 1)
        n[s] = max(1, min(n[s], L0[s] - first_own))
    case, ts = onehot_case(spec, seed, lambda s, c: int(rng.integers(0, c)),
                           max_pos=lambda s: int(L0[s] - n[s]))
    return case, onehot_queries(case, n), ts


def _onehot_want(case, qs, ts):
    """Row-by-row expected output: v_{t*} of the row's sequence (int8: code x
    scale as the oracle's write leaves it), repeated over the group's heads,
    in fp32 then rounded to the q dtype."""
    import pins
    from gpu_helpers import TORCH_DT
    if case.spec.cache == "i8":
        ok, ov = oracle.fill_cache(case)
        dense = pins.dense_kv(case, ok, ov)
    else:
        dense = pins.dense_kv(case)
    G = case.Hq // case.Hkv
    want = np.empty((qs.num_tokens, case.Hq, case.D), dtype=np.float64)
    for s, t in enumerate(ts):
        v = np.repeat(dense[s][1][t].astype(np.float32), G, axis=0)
        vq = torch.from_numpy(v).to(TORCH_DT[case.spec.act]).double().numpy()
        want[qs.query_start_loc[s]:qs.query_start_loc[s + 1]] = vq
    return want


@pytest.mark.parametrize("P", [0, 64])
@pytest.mark.parametrize("name", list(EXACT))
def test_prefill_onehot_bit_exact(name, P):
    """Through shuffled block tables, every query row of every sequence sees its
    sequence's probe token t* (placed at or before the first new token) and
    returns v_{t*} bit for bit: the block-table lookup and the K/V gather are
    exact, and the int8 path dequantises V exactly as the oracle does."""
    rng = np.random.default_rng(17)
    for rep in range(2):
        case, qs, ts = _onehot_prefill(name, 60 + rep, rng)
        print(f"[onehot prefill] {name} P={P} rep {rep}: {qs.num_tokens} rows", flush=True)
        dc = to_device(case)
        fill_pool(dc)
        got = run_prefill(case, qs, dc, partition_size=P)
        want = _onehot_want(case, qs, ts)
        bad = np.argwhere(got != want)
        assert bad.size == 0, f"{name} P={P}: first mismatch at row/head/dim {bad[0]}"


@pytest.mark.parametrize("name", ["g4_b16", "g4_b16_rows4", "g8_b32_cow", "g8_b32_cow_rows3",
                                  "g1_rows20", "g4_rows40"])
def test_write_prefill_onehot_bit_exact(name):
    """The fused write: the new tokens' slots hold poison before the call, t* may
    be a new token (read from key / value), and the output is v_{t*} bit for
    bit; the pool afterwards is byte-identical to the oracle's write."""
    rng = np.random.default_rng(19)
    case, qs, ts = _onehot_prefill(name, 70, rng)
    ok, ov = oracle.fill_cache(case)
    kn, vn, slots = new_token_rows(case, qs)
    kp, vp = ok.copy(), ov.copy()
    for arr in (kp, vp):
        arr.reshape(case.num_blocks, case.Hkv, case.B, case.D)[
            slots // case.B, :, slots % case.B, :] = synth.BF16_POISON
    k = host_to_dev(kp, "bf16", "cuda")
    v = host_to_dev(vp, "bf16", "cuda")
    dc = to_device(case)
    q = host_to_dev(qs.q, "bf16", "cuda")
    qsl = torch.from_numpy(qs.query_start_loc).cuda()
    out = torch.full_like(q, float("nan"))
    pa.write_prefill(host_to_dev(kn, "bf16", "cuda"), host_to_dev(vn, "bf16", "cuda"),
                     torch.from_numpy(slots).cuda(), out, q, k, v, dc.block_tables,
                     dc.context_lens, qsl, float(case.scale), int(qs.q_lens.max()),
                     case.max_context_len)
    torch.cuda.synchronize()
    from gpu_helpers import dev_to_host
    assert np.array_equal(dev_to_host(k).view(np.uint8), ok.view(np.uint8)), "K pool differs"
    assert np.array_equal(dev_to_host(v).view(np.uint8), ov.view(np.uint8)), "V pool differs"
    assert np.array_equal(as_f64(out), _onehot_want(case, qs, ts))


@pytest.mark.parametrize("cache", ["bf16", "i8"])
@pytest.mark.parametrize("P", [0, 32])
def test_prefill_context_len_one_returns_v(cache, P):
    """Every context is the new token alone: the output is its V row exactly
    (int8: its codes times the block's V scale, in fp32, then rounded)."""
    spec = synth.CONFIGS[2 if cache == "bf16" else 4].replace(
        num_seqs=24, lens=("const", 1), max_len=16)
    case = synth.make_case(spec, 9)
    qs = synth.Queries(query_start_loc=np.arange(case.S + 1, dtype=np.int32), q=case.q,
                       q_lens=np.ones(case.S, dtype=np.int64))
    dc = to_device(case)
    fill_pool(dc)
    got = run_prefill(case, qs, dc, partition_size=P)
    assert np.array_equal(got, _onehot_want(case, qs, [0] * case.S))


def test_write_prefill_context_len_one_returns_v():
    spec = synth.CONFIGS[5].replace(num_seqs=32, lens=("const", 1), max_len=32,
                                    prefix_groups=0, prefix_tokens=0)
    case = synth.make_case(spec, 10)
    from gpu_helpers import poison_pool, dev_to_host
    dc = to_device(case)
    k, v = poison_pool(case)
    qsl = torch.arange(case.S + 1, dtype=torch.int32, device="cuda")
    out = torch.full_like(dc.q, float("nan"))
    pa.write_prefill(dc.key, dc.value, dc.slot_mapping, out, dc.q, k, v, dc.block_tables,
                     dc.context_lens, qsl, float(case.scale), 1, case.max_context_len)
    torch.cuda.synchronize()
    G = case.Hq // case.Hkv
    assert np.array_equal(dev_to_host(out), np.repeat(case.value, G, axis=1))
    ok, ov = oracle.fill_cache(case)
    assert np.array_equal(dev_to_host(k).view(np.uint8), ok.view(np.uint8))


@pytest.mark.parametrize("name", ["g4_b16", "g4_b16_rows4", "g8_b32_cow_rows3", "g4_i8_b16_rows4",
                                  "g4_rows40"])
def test_prefill_placement_bit_identical(name):
    """Renaming the physical blocks, and un-sharing copy-on-write prefixes, leave
    the output bit-identical, in one pass and split over 64-token partitions
    (the arithmetic order depends only on logical positions)."""
    spec, rows = EXACT[name]
    case = synth.make_case(spec, 80)
    qs = synth.make_queries(case, ("const", rows), 81)
    variants = [synth.permute_placement(case, 82), synth.permute_placement(case, 83)]
    if spec.prefix_groups:
        variants.append(synth.unshare_prefixes(case))
    base = []
    dc = to_device(case)
    fill_pool(dc)
    for P in (0, 64):
        base.append(run_prefill(case, qs, dc, partition_size=P))
    for var in variants:
        dv = to_device(var)
        fill_pool(dv)
        for P, b in zip((0, 64), base):
            assert np.array_equal(run_prefill(var, qs, dv, partition_size=P), b), f"P={P}"


@pytest.mark.parametrize("name", ["verify_g4", "mixed_g4", "cow_g8", "decode_ties_s64",
                                  "verify_g4_i8", "g2_i8_b32"])
def test_write_prefill_negative_slots_match_two_calls(name):
    """New tokens with a negative slot are neither written nor read from key /
    value: the fused launch stays bit-identical (output and pool) to
    pa_write_kv_cache followed by pa_prefill, whose decode then reads whatever
    the cache holds at those positions."""
    case, qs, dc = prepare(name)
    if name == "cow_g8":
        qs = synth.make_queries(case, ("const", 1), 12)
    kn, vn, slots = new_token_rows(case, qs)
    slots = slots.copy()
    slots[::3] = -1
    args = (host_to_dev(kn, "bf16", "cuda"), host_to_dev(vn, "bf16", "cuda"),
            torch.from_numpy(slots).cuda())
    q = host_to_dev(qs.q, "bf16", "cuda")
    qsl = torch.from_numpy(qs.query_start_loc).cuda()
    mq, maxL = int(qs.q_lens.max()), case.max_context_len
    ks, vs = dc.k_scale, dc.v_scale
    for P in (0, 64):
        k1, v1 = dc.k_cache.clone(), dc.v_cache.clone()
        k2, v2 = dc.k_cache.clone(), dc.v_cache.clone()
        # the skipped positions hold other values in the cache than in key / value
        # (bf16: one mantissa ulp; int8: one code)
        iv = torch.int8 if case.spec.cache == "i8" else torch.int16
        for kk, vv in ((k1, v1), (k2, v2)):
            kk.view(iv).bitwise_xor_(1)
            vv.view(iv).bitwise_xor_(1)
        a = torch.empty_like(q)
        b = torch.empty_like(q)
        if P:
            w1 = pa.prefill_workspace(qs.num_tokens, case.Hq, case.D, maxL, P, "cuda")
            w2 = pa.prefill_workspace(qs.num_tokens, case.Hq, case.D, maxL, P, "cuda")
            pa.write_prefill(*args, None, q, k1, v1, dc.block_tables, dc.context_lens, qsl,
                             float(case.scale), mq, maxL, ks, vs, partition_size=P,
                             tmp_out=w1[0], tmp_max=w1[1], tmp_sum=w1[2], row_lens=w1[3])
            pa.decode_splitk_reduce(a, w1[0], w1[1], w1[2], w1[3], maxL, P)
            pa.write_kv_cache(args[0], args[1], k2, v2, args[2], ks, vs)
            pa.prefill(None, q, k2, v2, dc.block_tables, dc.context_lens, qsl,
                       float(case.scale), mq, maxL, ks, vs, partition_size=P, tmp_out=w2[0],
                       tmp_max=w2[1], tmp_sum=w2[2], row_lens=w2[3])
            pa.decode_splitk_reduce(b, w2[0], w2[1], w2[2], w2[3], maxL, P)
        else:
            pa.write_prefill(*args, a, q, k1, v1, dc.block_tables, dc.context_lens, qsl,
                             float(case.scale), mq, maxL, ks, vs)
            pa.write_kv_cache(args[0], args[1], k2, v2, args[2], ks, vs)
            pa.prefill(b, q, k2, v2, dc.block_tables, dc.context_lens, qsl, float(case.scale),
                       mq, maxL, ks, vs)
        torch.cuda.synchronize()
        assert torch.equal(k1.view(iv), k2.view(iv)), f"P={P}: K pool"
        assert torch.equal(v1.view(iv), v2.view(iv)), f"P={P}: V pool"
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"P={P}: output"
