"""HIP path (through the C ABI) against the fp64 oracle, on the GPU.

Bars: the slot-mapped write is byte-exact over the whole pool (every slot,
including untouched poison); one-hot probes, L = 1 and placement changes are
bit-exact; decode outputs are within max |GPU - oracle| <= 1e-5 (fp32),
2e-2 (bf16) and 3e-2 (int8 KV, same dequantisation on both sides).
Small cases span several 16-token chunks, several partitions and a ragged
tail; the full-size workloads run in the bench's launch configuration and are
checked on sampled sequences (every head and dim of those sequences).
"""
import os

import numpy as np
import pytest
import torch

import oracle
import pins
import synth
from probe_cases import onehot_case
from gpu_helpers import (TORCH_DT, as_f64, dev_to_host, fill_pool, host_to_dev, poison_pool,
                         run_decode, to_device, tol)

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import paged_kv_decode_03_amd as pa

C = synth.CONFIGS
SMALL = {
    "cfg1": C[1],
    "cfg2s": C[2].replace(num_seqs=12, lens=("uniform", 1, 1100), max_len=1100),
    "cfg3s": C[3].replace(num_seqs=2, lens=("const", 4099), max_len=4099),
    "cfg4s": C[4].replace(num_seqs=10, lens=("uniform", 1, 1300), max_len=1300),
    "cfg5s": C[5].replace(num_seqs=16, lens=("lognormal", 200, 1.0, 1, 1500), max_len=1500,
                          prefix_groups=2, prefix_tokens=256),
    "mha_bf16_d128": synth.Spec("mha bf16", 6, ("uniform", 1, 700), 8, 8, 128, 16, act="bf16",
                                cache="bf16", max_len=700),
    "g2_bf16": synth.Spec("G=2 bf16", 6, ("uniform", 1, 600), 8, 4, 128, 32, act="bf16",
                          cache="bf16", max_len=600),
    "mha_i8_f32q": synth.Spec("MHA int8, fp32 q", 5, ("uniform", 1, 500), 4, 4, 64, 16,
                              act="f32", cache="i8", max_len=500),
    "mha_bf16_d64": synth.Spec("MHA bf16 D64", 5, ("uniform", 1, 500), 4, 4, 64, 32, act="bf16",
                               cache="bf16", max_len=500),
    "g8_i8": synth.Spec("G=8 int8", 6, ("uniform", 1, 900), 32, 4, 128, 16, act="bf16",
                        cache="i8", max_len=900),
    "g4_b32": synth.Spec("G=4 B=32", 6, ("uniform", 1, 900), 16, 4, 128, 32, act="bf16",
                         cache="bf16", max_len=900),
    "mha_f32_d128_b32": synth.Spec("MHA fp32 D128 B32", 4, ("uniform", 1, 400), 2, 2, 128, 32,
                                   act="f32", cache="f32", max_len=400),
    "g2_i8_bf16q": synth.Spec("G=2 int8", 4, ("uniform", 1, 400), 4, 2, 64, 16, act="bf16",
                              cache="i8", max_len=400),
    # 8 query heads per kv head on a bf16 cache: the balanced kernel takes pairs
    # of sequences; an odd count leaves the last pair without a second, and one
    # copy-on-write group makes most pairs share their leading blocks
    "g8_odd_cow": synth.Spec("G=8 bf16 CoW, odd count", 7, ("uniform", 1, 700), 64, 8, 128, 16,
                             act="bf16", cache="bf16", max_len=700, prefix_groups=1,
                             prefix_tokens=256),
    # groups of three: every other pair straddles two groups and shares nothing
    "g8_cow_g3": synth.Spec("G=8 bf16 CoW, groups of 3", 15, ("uniform", 1, 900), 64, 8, 128,
                            32, act="bf16", cache="bf16", max_len=900, prefix_groups=5,
                            prefix_tokens=256),
}

# Batches of 20k-30k 16-token chunks over all kv heads: every wave of the
# balanced schedule's persistent grid gets a range of several chunks, so most
# contexts are cut into several pieces that go through the in-kernel combine.
MID = {
    "mid_g4_bf16": synth.Spec("G=4 bf16, mid-size", 24, ("uniform", 1000, 3000), 32, 8, 128,
                              16, act="bf16", cache="bf16", max_len=3000),
    "mid_g8_i8": synth.Spec("G=8 int8, mid-size", 16, ("uniform", 1500, 3500), 64, 8, 128, 32,
                            act="bf16", cache="i8", max_len=3500),
    "mid_g8_cow": synth.Spec("G=8 bf16 CoW, mid-size", 48, ("lognormal", 800, 1.0, 1, 6000),
                             64, 8, 128, 32, act="bf16", cache="bf16", max_len=6000,
                             prefix_groups=4, prefix_tokens=512),
    # around the balanced kernel's pair table (2048 pair units): 4096 sequences
    # fill it, 4097 take the kernel with one sequence per segment
    "many_g8_4096": synth.Spec("G=8 bf16, 4096 sequences", 4096, ("uniform", 1, 48), 64, 8,
                               128, 16, act="bf16", cache="bf16", max_len=48,
                               prefix_groups=64, prefix_tokens=16),
    "many_g8_4097": synth.Spec("G=8 bf16, 4097 sequences", 4097, ("uniform", 1, 48), 64, 8,
                               128, 16, act="bf16", cache="bf16", max_len=48,
                               prefix_groups=17, prefix_tokens=16),
}

_cache = {}


def prepared(name, seed=7):
    """(case, device case with filled pool, oracle pool, oracle output)."""
    key = (name, seed)
    if key not in _cache:
        case = synth.make_case(SMALL[name] if name in SMALL else MID[name], seed)
        dc = to_device(case)
        fill_pool(dc)
        ok, ov = oracle.fill_cache(case)
        ref = oracle.decode_case(case, ok, ov)
        _cache[key] = (case, dc, ok, ov, ref)
    return _cache[key]


def sync():
    torch.cuda.synchronize()


# ---- write ------------------------------------------------------------------

@pytest.mark.parametrize("name", list(SMALL))
def test_write_pool_byte_exact(name):
    print(f"[write] {name}", flush=True)
    case, dc, ok, ov, _ = prepared(name)
    sync()
    assert np.array_equal(dev_to_host(dc.k_cache).view(np.uint8), ok.view(np.uint8)), "k pool"
    assert np.array_equal(dev_to_host(dc.v_cache).view(np.uint8), ov.view(np.uint8)), "v pool"


def test_write_skips_negative_slots():
    case = synth.make_case(SMALL["cfg4s"], 3)
    dc = to_device(case)
    k, v = poison_pool(case)
    slots = dc.slot_mapping.clone()
    slots[::2] = -1
    pa.write_kv_cache(dc.key, dc.value, k, v, slots, dc.k_scale, dc.v_scale)
    ok, ov = case.empty_pool()
    oracle.write_kv_cache(case.key, case.value, ok, ov, slots.cpu().numpy(), case.k_scale,
                          case.v_scale)
    sync()
    assert np.array_equal(dev_to_host(k), ok) and np.array_equal(dev_to_host(v), ov)


def test_write_int8_near_ties():
    """Quotients within half an fp32 ulp of a half-integer (double-rounding traps)."""
    pairs = pins.near_tie_pairs()
    n = len(pairs)
    x = np.array([p[0] for p in pairs], np.float32)
    for act in ("f32", "bf16"):
        key = (synth.bf16_bits(x) if act == "bf16" else x).reshape(n, 1, 1)
        key8 = np.repeat(key, 8, axis=2)                      # head_dim 8
        ks = np.array([p[1] for p in pairs], np.float32).reshape(n, 1)
        slots = np.arange(n, dtype=np.int64)
        ok = np.full((n, 1, 1, 8), -128, np.int8)
        ov = ok.copy()
        oracle.write_kv_cache(key8, key8, ok, ov, slots, ks, ks)
        k = torch.full((n, 1, 1, 8), -128, dtype=torch.int8, device="cuda")
        v = k.clone()
        kd = host_to_dev(key8, act, "cuda")
        pa.write_kv_cache(kd, kd, k, v, torch.from_numpy(slots).cuda(),
                          torch.from_numpy(ks).cuda(), torch.from_numpy(ks).cuda())
        sync()
        assert np.array_equal(dev_to_host(k), ok), act


# Scales across the quantiser's range: ordinary ones, and ones whose quotients
# reach the subnormal, overflow, zero, negative, infinite and NaN cases of the
# correctly rounded division.
INT8_SCALES = [1 / 127, 0.0123, 3.7e-3, 1.0, 0.125, 5.3e-5, 2.0 ** -125, 2.0 ** -126, 1e-39,
               2.0 ** 125, 2.0 ** 126, 3e38, 0.0, -0.37, float("inf"), float("nan")]


def _write_i8(key, value, slots, ks, vs, B, act):
    T, _, D = key.shape
    NB = ks.shape[0]
    k = torch.full((NB, 1, B, D), -128, dtype=torch.int8, device="cuda")
    v = k.clone()
    pa.write_kv_cache(host_to_dev(key, act, "cuda"), host_to_dev(value, act, "cuda"), k, v,
                      torch.from_numpy(slots).cuda(), torch.from_numpy(ks).cuda(),
                      torch.from_numpy(vs).cuda())
    ok = np.full((NB, 1, B, D), -128, np.int8)
    ov = ok.copy()
    oracle.write_kv_cache(key, value, ok, ov, slots, ks, vs)
    sync()
    return dev_to_host(k), dev_to_host(v), ok, ov


def test_write_int8_every_bf16_value():
    """All 65536 bf16 values through the int8 write at each scale, byte-exact."""
    D, B = 64, 16
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    T = bits.size // D
    key = bits.reshape(T, 1, D)
    value = key[::-1].copy()
    slots = np.arange(T, dtype=np.int64)
    for sc in INT8_SCALES:
        ks = np.full((T // B, 1), sc, np.float32)
        k, v, ok, ov = _write_i8(key, value, slots, ks, ks.copy(), B, "bf16")
        assert np.array_equal(k, ok) and np.array_equal(v, ov), sc


def test_write_int8_fp32_boundaries():
    """fp32 activations within 8 ulps of every rounding boundary k + 1/2 of
    the code range (and a little beyond), byte-exact."""
    D, B = 64, 16
    for sc in (np.float32(0.0123), np.float32(1 / 127), np.float32(3.0), np.float32(2.0 ** -10)):
        base = ((np.arange(-130, 130) + 0.5) * np.float64(sc)).astype(np.float32)
        steps = np.arange(-8, 9, dtype=np.int32)
        xs = (base.view(np.int32)[:, None] + steps[None, :]).reshape(-1).view(np.float32)
        T = -(-xs.size // D)
        T = -(-T // B) * B
        key = np.zeros(T * D, np.float32)
        key[:xs.size] = xs
        key = key.reshape(T, 1, D)
        value = -key
        slots = np.arange(T, dtype=np.int64)
        ks = np.full((T // B, 1), sc, np.float32)
        k, v, ok, ov = _write_i8(key, value, slots, ks, ks.copy(), B, "f32")
        assert np.array_equal(k, ok) and np.array_equal(v, ov), float(sc)


# ---- decode -----------------------------------------------------------------

PARITY = [(n, 0) for n in SMALL] + [
    ("cfg1", 16), ("cfg1", 32), ("cfg1", 112),
    ("cfg2s", 64), ("cfg2s", 512), ("cfg2s", 2048),
    ("cfg3s", 512), ("cfg3s", 256),
    ("cfg4s", 128), ("cfg4s", 512),
    ("cfg5s", 64), ("cfg5s", 512),
    ("mha_bf16_d128", 128), ("g2_bf16", 96), ("mha_i8_f32q", 64), ("mha_bf16_d64", 64),
    ("g8_i8", 256), ("g4_b32", 160), ("mha_f32_d128_b32", 96), ("g2_i8_bf16q", 48),
]


@pytest.mark.parametrize("name,P", PARITY)
def test_decode_parity(name, P):
    print(f"[decode] {name} P={P}", flush=True)
    case, dc, ok, ov, ref = prepared(name)
    out = run_decode(dc, P)
    sync()
    got = as_f64(out)
    assert np.isfinite(got).all(), "non-finite output (poison leaked?)"
    err = np.abs(got - ref).max()
    assert err <= tol(case), f"{name} P={P}: max |gpu - oracle| = {err}"


@pytest.mark.parametrize("name", ["cfg1", "cfg2s", "cfg5s", "g8_i8"])
def test_splitk_partials(name):
    """Each partition's (o_j, m_j, l_j) against the oracle's partials. With a
    bf16 cache the MFMA kernel rounds each weight to bf16 before PV and sums the
    rounded weights into l_j, so l_j is within the bf16 unit roundoff (2^-9,
    bound here by 2^-8 with the fp32 sums) of the exact sum; fp32 weights are
    within 1e-4."""
    case, dc, ok, ov, _ = prepared(name)
    P = 64
    S, Hq, D = case.S, case.Hq, case.D
    ws = pa.workspace(S, Hq, D, case.max_context_len, P, "cuda")
    for t in ws:
        t.fill_(float("nan"))
    pa.decode(None, dc.q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens,
              float(case.scale), case.max_context_len, P, *ws, k_scale=dc.k_scale,
              v_scale=dc.v_scale)
    o, m, l = oracle.decode_partials(case.q, ok, ov, case.block_tables, case.context_lens,
                                     case.scale, P, case.k_scale, case.v_scale)
    sync()
    go, gm, gl = (t.cpu().numpy().astype(np.float64) for t in ws)
    n = -(-case.context_lens.astype(np.int64) // P)
    l_tol = 2.0 ** -8 if case.spec.cache == "bf16" else 1e-4
    for s in range(S):
        assert np.isnan(go[s, :, n[s]:]).all(), "partition past the length was written"
        sl = slice(0, n[s])
        assert np.abs(go[s, :, sl] - o[s, :, sl]).max() <= tol(case)
        assert np.abs(gm[s, :, sl] - m[s, :, sl]).max() <= 1e-4 * max(1.0, np.abs(m[s, :, sl]).max())
        assert np.abs(gl[s, :, sl] / l[s, :, sl] - 1).max() <= l_tol


def test_reduce_from_oracle_partials():
    """pa_decode_splitk_reduce fed the oracle's partials (rounded to fp32)."""
    case = synth.make_case(SMALL["cfg2s"], 5)
    ok, ov = oracle.fill_cache(case)
    P = 128
    o, m, l = oracle.decode_partials(case.q, ok, ov, case.block_tables, case.context_lens,
                                     case.scale, P)
    o32, m32, l32 = (np.nan_to_num(a, nan=0.0).astype(np.float32) for a in (o, m, l))
    want = oracle.splitk_reduce(o32.astype(np.float64), m32.astype(np.float64),
                                l32.astype(np.float64), case.context_lens, P)
    for dt, tl in ((torch.float32, 1e-5), (torch.bfloat16, 1e-2)):
        out = torch.empty((case.S, case.Hq, case.D), dtype=dt, device="cuda")
        pa.decode_splitk_reduce(out, torch.from_numpy(o32).cuda(), torch.from_numpy(m32).cuda(),
                                torch.from_numpy(l32).cuda(),
                                torch.from_numpy(case.context_lens).cuda(),
                                case.max_context_len, P)
        sync()
        assert np.abs(as_f64(out) - want).max() <= tl


@pytest.mark.parametrize("P", [16, 128])
def test_reduce_ignores_partials_past_the_length(P):
    """The reduce loads the first partitions of every row before it knows the
    row's own partition count; those past it hold NaN here and must not
    reach the output. P = 16: up to 69 partitions, so the later rounds of
    the combine (past the first four per wave) run as well."""
    case = synth.make_case(SMALL["cfg2s"], 5)
    ok, ov = oracle.fill_cache(case)
    o, m, l = oracle.decode_partials(case.q, ok, ov, case.block_tables, case.context_lens,
                                     case.scale, P)
    n = -(-case.context_lens.astype(np.int64) // P)
    assert n.max() > 16 or P == 128
    o32, m32, l32 = (a.astype(np.float32) for a in (o, m, l))
    for s in range(case.S):                            # past the length: NaN (the oracle's)
        assert np.isnan(o32[s, :, n[s]:]).all() and np.isnan(m32[s, :, n[s]:]).all()
    want = oracle.splitk_reduce(np.nan_to_num(o32, nan=0.0).astype(np.float64),
                                np.nan_to_num(m32, nan=0.0).astype(np.float64),
                                np.nan_to_num(l32, nan=0.0).astype(np.float64),
                                case.context_lens, P)
    out = torch.empty((case.S, case.Hq, case.D), dtype=torch.float32, device="cuda")
    pa.decode_splitk_reduce(out, torch.from_numpy(o32).cuda(), torch.from_numpy(m32).cuda(),
                            torch.from_numpy(l32).cuda(), torch.from_numpy(case.context_lens).cuda(),
                            case.max_context_len, P)
    sync()
    got = as_f64(out)
    assert np.isfinite(got).all()
    assert np.abs(got - want).max() <= 1e-5


# ---- exactness ----------------------------------------------------------------

def _onehot_case(spec, seed, tstar_of):
    """q = 128 e_0, k_{t*} = 128 e_0, other k_0 = 0: the output is v_{t*} exactly."""
    return onehot_case(spec, seed, tstar_of)


@pytest.mark.parametrize("name", ["cfg1", "cfg2s", "cfg4s", "cfg5s", "g2_bf16", "mha_i8_f32q"])
@pytest.mark.parametrize("P", [0, 64])
def test_onehot_bit_exact(name, P):
    spec = SMALL[name]
    rng = np.random.default_rng(11)
    for rep in range(3):
        case, ts = _onehot_case(spec, 20 + rep, lambda s, L: int(rng.integers(0, L)))
        dc = to_device(case)
        fill_pool(dc)
        out = run_decode(dc, P)
        sync()
        got = as_f64(out)
        G = case.Hq // case.Hkv
        if spec.cache == "i8":
            # the oracle's write fixes the dequantised row: codes * scale
            ok, ov = oracle.fill_cache(case)
            dense = pins.dense_kv(case, ok, ov)
        else:
            dense = pins.dense_kv(case)
        for s, t in enumerate(ts):
            # float caches: v_{t*} itself; int8: the fp32 product code * scale
            want = np.repeat(dense[s][1][t].astype(np.float32), G, axis=0)
            want_q = torch.from_numpy(want).to(TORCH_DT[spec.act])
            assert np.array_equal(got[s], want_q.double().numpy()), f"{name} seq {s} t*={t}"


@pytest.mark.parametrize("spec", [
    synth.Spec("L1 f32", 6, ("const", 1), 4, 4, 64, 16, act="f32", cache="f32", max_len=16),
    synth.Spec("L1 bf16 G4", 6, ("const", 1), 32, 8, 128, 16, act="bf16", cache="bf16",
               max_len=16),
    synth.Spec("L1 bf16 G8", 6, ("const", 1), 64, 8, 128, 32, act="bf16", cache="bf16",
               max_len=32),
    synth.Spec("L1 bf16 G1", 6, ("const", 1), 8, 8, 128, 16, act="bf16", cache="bf16",
               max_len=16),
], ids=lambda s: s.name)
@pytest.mark.parametrize("split", [False, True])
def test_context_len_one_returns_v(spec, split):
    case = synth.make_case(spec, 9)
    dc = to_device(case)
    fill_pool(dc)
    out = run_decode(dc, case.B if split else 0)
    sync()
    G = case.Hq // case.Hkv
    want = np.repeat(case.value, G, axis=1)
    assert np.array_equal(dev_to_host(out), want)


@pytest.mark.parametrize("name", ["cfg1", "cfg2s", "cfg4s", "cfg5s", "g2_bf16"])
def test_placement_invariance_bit_identical(name):
    case, dc, _, _, _ = prepared(name)
    base = dev_to_host(run_decode(dc, 0))
    base_split = dev_to_host(run_decode(dc, 64))
    variants = [synth.permute_placement(case, 31), synth.permute_placement(case, 32)]
    if case.spec.prefix_groups:
        variants.append(synth.unshare_prefixes(case))
    for var in variants:
        dv = to_device(var)
        fill_pool(dv)
        assert np.array_equal(dev_to_host(run_decode(dv, 0)), base)
        assert np.array_equal(dev_to_host(run_decode(dv, 64)), base_split)


def test_deterministic_repeat():
    case, dc, _, _, _ = prepared("cfg5s")
    a = dev_to_host(run_decode(dc, 64))
    b = dev_to_host(run_decode(dc, 64))
    assert np.array_equal(a, b)


@pytest.mark.parametrize("name", ["cfg1", "cfg2s", "cfg4s"])
def test_zero_length_gives_zeros(name):
    case, dc, ok, ov, ref = prepared(name)
    lens = dc.context_lens.clone()
    lens[1] = 0
    for P in (0, 64):
        out = torch.full_like(dc.q, float("nan"))
        if P == 0:
            pa.decode(out, dc.q, dc.k_cache, dc.v_cache, dc.block_tables, lens, float(case.scale),
                      case.max_context_len, 0, k_scale=dc.k_scale, v_scale=dc.v_scale)
        else:
            ws = pa.workspace(case.S, case.Hq, case.D, case.max_context_len, P, "cuda")
            pa.decode(None, dc.q, dc.k_cache, dc.v_cache, dc.block_tables, lens,
                      float(case.scale), case.max_context_len, P, *ws, k_scale=dc.k_scale,
                      v_scale=dc.v_scale)
            pa.decode_splitk_reduce(out, *ws, lens, case.max_context_len, P)
        sync()
        got = as_f64(out)
        assert (got[1] == 0).all()
        keep = [s for s in range(case.S) if s != 1]
        assert np.abs(got[keep] - ref[keep]).max() <= tol(case)


def test_pa_check_rejects_bad_block_id(monkeypatch):
    """PA_CHECK=1 validates device indices on the host: a block id past the
    pool is reported and nothing is launched."""
    case, dc, _, _, _ = prepared("cfg1")
    bt = dc.block_tables.clone()
    bt[0, 0] = case.num_blocks + 5
    monkeypatch.setenv("PA_CHECK", "1")
    out = torch.empty_like(dc.q)
    with pytest.raises(pa.PAError) as e:
        pa.decode(out, dc.q, dc.k_cache, dc.v_cache, bt, dc.context_lens, float(case.scale),
                  case.max_context_len, 0)
    assert e.value.status == -7
    bad = dc.slot_mapping.clone()
    bad[0] = case.num_blocks * case.B + 3
    with pytest.raises(pa.PAError):
        pa.write_kv_cache(dc.key, dc.value, dc.k_cache.clone(), dc.v_cache.clone(), bad)


# ---- work-balanced schedule (pa_decode_balanced) ----------------------------------

BALANCED = [(n, 16) for n in SMALL] + [(n, 64) for n in SMALL] + [
    ("cfg2s", 256), ("cfg3s", 512), ("cfg4s", 512), ("cfg5s", 256), ("g8_i8", 128),
    ("cfg1", 112)]


@pytest.mark.parametrize("name,P", BALANCED)
def test_balanced_parity(name, P):
    """Pieces of >= P tokens; P = 16 cuts contexts into many pieces, so most
    outputs go through the cross-workgroup combine."""
    print(f"[balanced] {name} P={P}", flush=True)
    case, dc, ok, ov, ref = prepared(name)
    ws = pa.balanced_workspace(case.S, case.Hq, case.Hkv, case.D, case.max_context_len, P,
                               "cuda")
    out1 = run_decode(dc, P, ws=ws, balanced=True)
    out2 = run_decode(dc, P, ws=ws, balanced=True)        # counters must be back at zero
    sync()
    assert int(ws[3].abs().sum()) == 0, "counters not reset"
    got = as_f64(out1)
    assert np.isfinite(got).all()
    err = np.abs(got - ref).max()
    assert err <= tol(case), f"{name} P={P}: max |gpu - oracle| = {err}"
    assert np.array_equal(dev_to_host(out1), dev_to_host(out2)), "repeat not bit-identical"


@pytest.mark.parametrize("name", ["cfg1", "cfg2s", "cfg4s", "cfg5s", "g2_bf16", "mha_i8_f32q"])
@pytest.mark.parametrize("P", [16, 256])
def test_balanced_onehot_bit_exact(name, P):
    spec = SMALL[name]
    rng = np.random.default_rng(13)
    for rep in range(2):
        case, ts = _onehot_case(spec, 40 + rep, lambda s, L: int(rng.integers(0, L)))
        dc = to_device(case)
        fill_pool(dc)
        got = as_f64(run_decode(dc, P, balanced=True))
        sync()
        G = case.Hq // case.Hkv
        if spec.cache == "i8":
            ok, ov = oracle.fill_cache(case)
            dense = pins.dense_kv(case, ok, ov)
        else:
            dense = pins.dense_kv(case)
        for s, t in enumerate(ts):
            want = np.repeat(dense[s][1][t].astype(np.float32), G, axis=0)
            want_q = torch.from_numpy(want).to(TORCH_DT[spec.act])
            assert np.array_equal(got[s], want_q.double().numpy()), f"{name} seq {s} t*={t}"


@pytest.mark.parametrize("name", ["cfg1", "cfg2s", "cfg5s", "g4_b32"])
def test_balanced_placement_invariance(name):
    """Renaming physical blocks gives a bit-identical output. Un-sharing the
    copy-on-write prefixes changes the schedule itself (the balanced decode
    orders its work kv head major when sequences share first blocks), so the
    contexts are cut elsewhere and the split-K combination rounds differently:
    that output is checked against the oracle and the shared one to tolerance."""
    case, dc, _, _, ref = prepared(name)
    base = dev_to_host(run_decode(dc, 32, balanced=True))
    dv = to_device(synth.permute_placement(case, 41))
    fill_pool(dv)
    assert np.array_equal(dev_to_host(run_decode(dv, 32, balanced=True)), base)
    if case.spec.prefix_groups:
        dv = to_device(synth.unshare_prefixes(case))
        fill_pool(dv)
        got = as_f64(run_decode(dv, 32, balanced=True))
        assert np.abs(got - ref).max() <= tol(case)
        assert np.abs(got - as_f64(run_decode(dc, 32, balanced=True))).max() <= tol(case)


@pytest.mark.parametrize("name", ["cfg1", "cfg2s", "cfg4s", "cfg5s", "g8_odd_cow", "g8_cow_g3"])
def test_balanced_zero_lengths(name):
    """Empty contexts anywhere in the batch (first, middle, last) give zeros and
    do not disturb the pieces of their neighbours."""
    case, dc, ok, ov, ref = prepared(name)
    lens = dc.context_lens.clone()
    zero = sorted({0, case.S // 2, case.S - 1})
    lens[zero] = 0
    ws = pa.balanced_workspace(case.S, case.Hq, case.Hkv, case.D, case.max_context_len, 16,
                               "cuda")
    out = torch.full_like(dc.q, float("nan"))
    pa.decode_balanced(out, dc.q, dc.k_cache, dc.v_cache, dc.block_tables, lens,
                       float(case.scale), case.max_context_len, 16, *ws, k_scale=dc.k_scale,
                       v_scale=dc.v_scale)
    sync()
    got = as_f64(out)
    assert (got[zero] == 0).all()
    keep = [s for s in range(case.S) if s not in zero]
    assert np.abs(got[keep] - ref[keep]).max() <= tol(case)
    assert int(ws[3].abs().sum()) == 0


@pytest.mark.parametrize("P", [16, 64])
@pytest.mark.parametrize("name", list(MID))
def test_balanced_mid_size(name, P):
    """Every output against the oracle, repeats bit-identical, and every
    counter back at zero."""
    print(f"[mid] {name} P={P}", flush=True)
    case, dc, ok, ov, ref = prepared(name)
    ws = pa.balanced_workspace(case.S, case.Hq, case.Hkv, case.D, case.max_context_len, P,
                               "cuda")
    a = dev_to_host(run_decode(dc, P, ws=ws, balanced=True))
    assert int(ws[3].abs().sum()) == 0, "counters not reset"
    b = dev_to_host(run_decode(dc, P, ws=ws, balanced=True))
    assert int(ws[3].abs().sum()) == 0, "counters not reset"
    assert np.array_equal(a, b)
    got = as_f64(run_decode(dc, P, ws=ws, balanced=True))
    err = np.abs(got - ref).max()
    print(f"[mid] {name} P={P} max err {err:.3e}", flush=True)
    assert err <= tol(case)


def test_balanced_all_empty():
    case, dc, _, _, _ = prepared("cfg2s")
    lens = torch.zeros_like(dc.context_lens)
    ws = pa.balanced_workspace(case.S, case.Hq, case.Hkv, case.D, case.max_context_len, 64,
                               "cuda")
    out = torch.full_like(dc.q, float("nan"))
    pa.decode_balanced(out, dc.q, dc.k_cache, dc.v_cache, dc.block_tables, lens,
                       float(case.scale), case.max_context_len, 64, *ws)
    sync()
    assert (as_f64(out) == 0).all()


# ---- full-size workloads, sampled ---------------------------------------------

@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_full_size_sampled(cfg):
    spec = C[cfg]
    print(f"[full] cfg{cfg} generating", flush=True)
    case = synth.make_case(spec, cfg)
    dc = to_device(case)
    print(f"[full] cfg{cfg} gpu write+decode P={spec.partition_size}", flush=True)
    fill_pool(dc)
    out = run_decode(dc, spec.partition_size)
    outb = run_decode(dc, spec.partition_size, balanced=True)
    outt = run_decode(dc, 64, balanced=True)         # pieces >= 64 tokens
    sync()
    got = as_f64(out)
    gotb = as_f64(outb)
    gott = as_f64(outt)
    assert np.isfinite(got).all() and np.isfinite(gotb).all() and np.isfinite(gott).all()
    print(f"[full] cfg{cfg} oracle", flush=True)
    ok, ov = oracle.fill_cache(case)
    assert np.array_equal(dev_to_host(dc.k_cache).view(np.uint8), ok.view(np.uint8))
    assert np.array_equal(dev_to_host(dc.v_cache).view(np.uint8), ov.view(np.uint8))
    L = case.context_lens
    rng = np.random.default_rng(cfg)
    seqs = sorted({int(np.argmax(L)), int(np.argmin(L)), 0, case.S - 1,
                   *[int(x) for x in rng.choice(case.S, size=2, replace=False)]})
    if cfg == 3:
        seqs = seqs[:2]
    ref = oracle.decode_case(case, ok, ov, seqs=seqs)
    err = np.abs(got[seqs] - ref).max()
    errb = np.abs(gotb[seqs] - ref).max()
    errt = np.abs(gott[seqs] - ref).max()
    print(f"[full] cfg{cfg} seqs {seqs} max err {err:.3e} (partitions) {errb:.3e} (balanced)"
          f" {errt:.3e} (balanced, 64-token pieces)", flush=True)
    assert err <= tol(case) and errb <= tol(case) and errt <= tol(case)


# ---- write + decode in one call (pa_write_decode_balanced) ------------------------

FUSED = ["cfg2s", "cfg3s", "cfg4s", "cfg5s", "g8_i8", "g4_b32", "mid_g4_bf16", "mid_g8_i8",
         "mid_g8_cow", "cfg1", "mha_bf16_d128", "g2_i8_bf16q", "many_g8_4096", "many_g8_4097"]


@pytest.mark.parametrize("name", FUSED)
def test_write_decode_matches_two_calls(name):
    """The new tokens' slots start as poison: the call must write them before any
    load of their chunk. Output and pool are bit-identical to pa_write_kv_cache
    followed by pa_decode_balanced (MFMA instances: one launch; the others fall
    back to the two kernels)."""
    print(f"[fused] {name}", flush=True)
    case, dc, ok, ov, ref = prepared(name)
    P = 64

    def pre_pool():
        k, v = poison_pool(case)
        if dc.pre_slots.numel():
            pa.write_kv_cache(dc.pre_key, dc.pre_value, k, v, dc.pre_slots, dc.k_scale,
                              dc.v_scale)
        return k, v

    # two calls
    k2, v2 = pre_pool()
    pa.write_kv_cache(dc.key, dc.value, k2, v2, dc.slot_mapping, dc.k_scale, dc.v_scale)
    ws2 = pa.balanced_workspace(case.S, case.Hq, case.Hkv, case.D, case.max_context_len, P, "cuda")
    out2 = torch.empty_like(dc.q)
    pa.decode_balanced(out2, dc.q, k2, v2, dc.block_tables, dc.context_lens, float(case.scale),
                       case.max_context_len, P, *ws2, k_scale=dc.k_scale, v_scale=dc.v_scale)
    # one call, twice (the second on a pool that already holds the tokens)
    k1, v1 = pre_pool()
    ws1 = pa.balanced_workspace(case.S, case.Hq, case.Hkv, case.D, case.max_context_len, P, "cuda")
    outs = []
    for _ in range(2):
        out1 = torch.full_like(dc.q, float("nan"))
        pa.write_decode_balanced(dc.key, dc.value, dc.slot_mapping, out1, dc.q, k1, v1,
                                 dc.block_tables, dc.context_lens, float(case.scale),
                                 case.max_context_len, P, *ws1, k_scale=dc.k_scale,
                                 v_scale=dc.v_scale)
        outs.append(out1)
    sync()
    assert int(ws1[3].abs().sum()) == 0, "counters not reset"
    assert np.array_equal(dev_to_host(k1).view(np.uint8), dev_to_host(k2).view(np.uint8))
    assert np.array_equal(dev_to_host(v1).view(np.uint8), dev_to_host(v2).view(np.uint8))
    assert np.array_equal(dev_to_host(k1).view(np.uint8), ok.view(np.uint8))
    want = dev_to_host(out2)
    for o in outs:
        assert np.array_equal(dev_to_host(o), want)
    err = np.abs(as_f64(outs[0]) - ref).max()
    print(f"[fused] {name} max err {err:.3e}", flush=True)
    assert err <= tol(case)


@pytest.mark.parametrize("name", ["cfg2s", "cfg4s", "cfg5s", "g8_i8", "mid_g8_cow"])
def test_write_decode_negative_slots_match_two_calls(name):
    """New tokens with a negative slot are not written: the fused call stays
    bit-identical (output and pool) to pa_write_kv_cache followed by
    pa_decode_balanced, which reads whatever the cache holds at position L - 1."""
    case, dc, ok, ov, ref = prepared(name)
    P = 64
    slots = dc.slot_mapping.clone()
    slots[::3] = -1
    k1, v1 = dc.k_cache.clone(), dc.v_cache.clone()
    k2, v2 = dc.k_cache.clone(), dc.v_cache.clone()
    for kk, vv in ((k1, v1), (k2, v2)):              # the cache differs from key / value
        kk.view(torch.uint8 if case.spec.cache == "i8" else torch.int16).bitwise_xor_(1)
        vv.view(torch.uint8 if case.spec.cache == "i8" else torch.int16).bitwise_xor_(1)
    ws1 = pa.balanced_workspace(case.S, case.Hq, case.Hkv, case.D, case.max_context_len, P, "cuda")
    ws2 = pa.balanced_workspace(case.S, case.Hq, case.Hkv, case.D, case.max_context_len, P, "cuda")
    a = torch.empty_like(dc.q)
    b = torch.empty_like(dc.q)
    pa.write_decode_balanced(dc.key, dc.value, slots, a, dc.q, k1, v1, dc.block_tables,
                             dc.context_lens, float(case.scale), case.max_context_len, P, *ws1,
                             k_scale=dc.k_scale, v_scale=dc.v_scale)
    pa.write_kv_cache(dc.key, dc.value, k2, v2, slots, dc.k_scale, dc.v_scale)
    pa.decode_balanced(b, dc.q, k2, v2, dc.block_tables, dc.context_lens, float(case.scale),
                       case.max_context_len, P, *ws2, k_scale=dc.k_scale, v_scale=dc.v_scale)
    sync()
    assert np.array_equal(dev_to_host(k1).view(np.uint8), dev_to_host(k2).view(np.uint8))
    assert np.array_equal(dev_to_host(v1).view(np.uint8), dev_to_host(v2).view(np.uint8))
    assert np.array_equal(dev_to_host(a), dev_to_host(b))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg", [4, 5])
def test_default_balanced_step_full_size_sampled(cfg):
    """The default decode step of the int8 batch and of the mixed copy-on-write
    batch at full size, in the exact launch configuration the bench times:
    pa_write_decode_balanced with pieces of >= 128 tokens writes every new token
    (its slot holds poison before) and decodes in one launch. The pool is
    byte-identical to the oracle's write; sampled sequences (every head and
    dim) are within tolerance of the oracle's decode; a second step on the
    same inputs is bit-identical and leaves the counters at zero."""
    spec = C[cfg]
    print(f"[default balanced] cfg{cfg}: generating", flush=True)
    case = synth.make_case(spec, cfg)
    dc = to_device(case)
    k, v = poison_pool(case)
    if dc.pre_slots.numel():
        pa.write_kv_cache(dc.pre_key, dc.pre_value, k, v, dc.pre_slots, dc.k_scale, dc.v_scale)
    P = 128
    ws = pa.balanced_workspace(case.S, case.Hq, case.Hkv, case.D, case.max_context_len, P,
                               "cuda")
    outs = []
    print(f"[default balanced] cfg{cfg}: gpu", flush=True)
    for _ in range(2):
        out = torch.full_like(dc.q, float("nan"))
        pa.write_decode_balanced(dc.key, dc.value, dc.slot_mapping, out, dc.q, k, v,
                                 dc.block_tables, dc.context_lens, float(case.scale),
                                 case.max_context_len, P, *ws, k_scale=dc.k_scale,
                                 v_scale=dc.v_scale)
        outs.append(out)
    sync()
    assert int(ws[3].abs().sum()) == 0, "counters not reset"
    assert np.array_equal(dev_to_host(outs[0]), dev_to_host(outs[1]))
    got = as_f64(outs[0])
    assert np.isfinite(got).all()
    print(f"[default balanced] cfg{cfg}: oracle", flush=True)
    ok, ov = oracle.fill_cache(case)
    assert np.array_equal(dev_to_host(k).view(np.uint8), ok.view(np.uint8)), "K pool differs"
    assert np.array_equal(dev_to_host(v).view(np.uint8), ov.view(np.uint8)), "V pool differs"
    L = case.context_lens
    rng = np.random.default_rng(cfg)
    seqs = sorted({int(np.argmax(L)), int(np.argmin(L)), 0, case.S - 1,
                   *[int(x) for x in rng.choice(case.S, size=4, replace=False)]})
    ref = oracle.decode_case(case, ok, ov, seqs=seqs)
    err = np.abs(got[seqs] - ref).max()
    print(f"[default balanced] cfg{cfg}: seqs {seqs} max err {err:.3e}", flush=True)
    assert err <= tol(case)
