"""pa_copy_blocks (through the C ABI) against the oracle's copy, on the GPU.

Bars: the whole K and V pools (every byte, poison included) and the int8
scales equal the oracle's after the same copies; a decode through tables
repointed at the copies is bit-identical to the decode before them (the GPU
path's arithmetic order depends only on logical positions)."""
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import dev_to_host, fill_pool, run_decode, to_device

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import paged_kv_decode_03_amd as pa

C = synth.CONFIGS
SPECS = {
    "cfg1_f32": C[1],
    "cfg2s_bf16": C[2].replace(num_seqs=12, lens=("uniform", 1, 1100), max_len=1100),
    "cfg4s_i8": C[4].replace(num_seqs=10, lens=("uniform", 1, 1300), max_len=1300),
    "cfg5s_cow": C[5].replace(num_seqs=16, lens=("lognormal", 200, 1.0, 1, 1500), max_len=1500,
                              prefix_groups=2, prefix_tokens=256),
}


def sync():
    torch.cuda.synchronize()


def cow_mapping(case, rng, extra=16):
    """(pairs, repointed block tables): each sequence's first shared block goes
    to a free block of its own (copy-on-write), plus `extra` used -> free copies."""
    B = case.B
    nblk = -(-case.context_lens.astype(np.int64) // B)
    used = sorted({int(b) for s in range(case.S) for b in case.block_tables[s, :nblk[s]]})
    free = [b for b in range(case.num_blocks) if b not in set(used) and b != case.poison_block]
    rng.shuffle(free)
    pairs, bt = [], case.block_tables.copy()
    for s in range(case.S):
        for lb in range(int(nblk[s])):
            b = int(bt[s, lb])
            if case.refcount[b] > 1 and free:
                d = free.pop()
                pairs.append((b, d))
                bt[s, lb] = d
                break
    srcs = {p for p, _ in pairs}
    for b in rng.choice(used, size=min(extra, len(used)), replace=False):
        if free and int(b) not in {d for _, d in pairs}:
            pairs.append((int(b), free.pop()))
    return np.array(pairs, dtype=np.int64).reshape(-1, 2), bt


@pytest.mark.parametrize("name", list(SPECS))
def test_copy_matches_oracle(name):
    print(f"[copy] {name}", flush=True)
    case = synth.make_case(SPECS[name], 13)
    dc = to_device(case)
    k, v = fill_pool(dc)
    ok, ov = oracle.fill_cache(case)
    assert np.array_equal(dev_to_host(k).view(np.uint8), ok.view(np.uint8))
    pairs, bt = cow_mapping(case, np.random.default_rng(1))
    assert len(pairs) >= 8
    ks = None if case.k_scale is None else case.k_scale.copy()
    vs = None if case.v_scale is None else case.v_scale.copy()
    oracle.copy_blocks(ok, ov, pairs, ks, vs)
    pa.copy_blocks(k, v, torch.from_numpy(pairs).cuda(), dc.k_scale, dc.v_scale)
    sync()
    assert np.array_equal(dev_to_host(k).view(np.uint8), ok.view(np.uint8)), "k pool"
    assert np.array_equal(dev_to_host(v).view(np.uint8), ov.view(np.uint8)), "v pool"
    if ks is not None:
        assert np.array_equal(dc.k_scale.cpu().numpy(), ks)
        assert np.array_equal(dc.v_scale.cpu().numpy(), vs)


@pytest.mark.parametrize("name", ["cfg5s_cow", "cfg4s_i8"])
def test_decode_after_copy_bit_identical(name):
    case = synth.make_case(SPECS[name], 14)
    dc = to_device(case)
    fill_pool(dc)
    before = dev_to_host(run_decode(dc, 0))
    pairs, bt = cow_mapping(case, np.random.default_rng(2))
    pa.copy_blocks(dc.k_cache, dc.v_cache, torch.from_numpy(pairs).cuda(), dc.k_scale,
                   dc.v_scale)
    dc.block_tables = torch.from_numpy(bt).cuda()
    after = dev_to_host(run_decode(dc, 0))
    sync()
    assert np.array_equal(before, after)


def test_many_pairs_and_empty():
    """Thousands of copies in one call (half the pool onto the other half), then
    an empty mapping."""
    spec = C[2].replace(num_seqs=48, lens=("uniform", 1000, 2048), max_len=2048)
    case = synth.make_case(spec, 15)
    dc = to_device(case)
    k, v = fill_pool(dc)
    ok, ov = oracle.fill_cache(case)
    rng = np.random.default_rng(3)
    ids = rng.permutation(case.num_blocks)
    n = case.num_blocks // 2
    assert n >= 2000
    pairs = np.stack([ids[:n], ids[n:2 * n]], axis=1).astype(np.int64)
    oracle.copy_blocks(ok, ov, pairs)
    pa.copy_blocks(k, v, torch.from_numpy(pairs).cuda())
    pa.copy_blocks(k, v, torch.zeros((0, 2), dtype=torch.int64, device="cuda"))
    sync()
    assert np.array_equal(dev_to_host(k).view(np.uint8), ok.view(np.uint8))
    assert np.array_equal(dev_to_host(v).view(np.uint8), ov.view(np.uint8))


def test_pa_check_rejects_bad_mapping(monkeypatch):
    """PA_CHECK=1 refuses a repeated destination before anything is enqueued."""
    case = synth.make_case(SPECS["cfg2s_bf16"], 16)
    dc = to_device(case)
    k, v = fill_pool(dc)
    before = dev_to_host(k).copy()
    monkeypatch.setenv("PA_CHECK", "1")
    bad = torch.tensor([[1, 5], [2, 5]], dtype=torch.int64, device="cuda")
    with pytest.raises(pa.PAError) as e:
        pa.copy_blocks(k, v, bad)
    assert e.value.status == -7
    sync()
    assert np.array_equal(dev_to_host(k), before)
