"""pa_write_decode_balanced_noalloc (workspace in the library's static per-GPU
array) against pa_write_decode_balanced with a caller-allocated workspace,
through the C ABI, on the GPU.

Bar: output and pool bit-identical to the allocating call on the same inputs,
and within the decode tolerance of the oracle; two calls in a row share the
one array, the second on a smaller batch, so leftover partials or counters of
the first would show in the second. Shapes beyond the array are refused
before anything is enqueued.
"""
import ctypes

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
    # MFMA instances (G = 4 and 8, bf16 and int8 caches, copy-on-write prefixes)
    "cow_g8_big": synth.Spec("G=8 bf16 CoW", 48, ("lognormal", 800, 1.0, 1, 6000), 64, 8, 128,
                             32, act="bf16", cache="bf16", max_len=6000, prefix_groups=4,
                             prefix_tokens=512),
    "cow_g8_small": C[5].replace(num_seqs=16, lens=("lognormal", 200, 1.0, 1, 1500),
                                 max_len=1500, prefix_groups=2, prefix_tokens=256),
    "i8_g8_big": synth.Spec("G=8 int8", 16, ("uniform", 1500, 3500), 64, 8, 128, 32, act="bf16",
                            cache="i8", max_len=3500),
    "i8_g4_small": C[4].replace(num_seqs=10, lens=("uniform", 1, 1300), max_len=1300),
    # VALU instances (G = 1 and 2)
    "mha_bf16_big": synth.Spec("MHA bf16", 6, ("uniform", 1, 700), 8, 8, 128, 16, act="bf16",
                               cache="bf16", max_len=700),
    "g2_i8_small": synth.Spec("G=2 int8", 4, ("uniform", 1, 400), 4, 2, 64, 16, act="bf16",
                              cache="i8", max_len=400),
    "g2_f32_d128": synth.Spec("G=2 fp32 D128", 8, ("uniform", 1, 900), 8, 4, 128, 32,
                              act="f32", cache="f32", max_len=900),
    "mha_i8_small": synth.Spec("MHA int8, fp32 q", 3, ("uniform", 1, 300), 4, 4, 64, 16,
                               act="f32", cache="i8", max_len=300),
}
PAIRS = [("cow_g8_big", "cow_g8_small"), ("i8_g8_big", "i8_g4_small"),
         ("mha_bf16_big", "g2_i8_small"), ("g2_f32_d128", "mha_i8_small")]


def pre_pool(case, dc):
    k, v = poison_pool(case)
    if dc.pre_slots.numel():
        pa.write_kv_cache(dc.pre_key, dc.pre_value, k, v, dc.pre_slots, dc.k_scale, dc.v_scale)
    return k, v


def step_both(case, dc, P):
    """The fused step on fresh pools (new-token slots hold poison): once with an
    allocated workspace, once without. Returns (out_alloc, out_noalloc, pools)."""
    ka, va = pre_pool(case, dc)
    kn, vn = pre_pool(case, dc)
    ws = pa.balanced_workspace(case.S, case.Hq, case.Hkv, case.D, case.max_context_len, P, "cuda")
    oa = torch.full_like(dc.q, float("nan"))
    on = torch.full_like(dc.q, float("nan"))
    pa.write_decode_balanced(dc.key, dc.value, dc.slot_mapping, oa, dc.q, ka, va,
                             dc.block_tables, dc.context_lens, float(case.scale),
                             case.max_context_len, P, *ws, k_scale=dc.k_scale, v_scale=dc.v_scale)
    pa.write_decode_balanced_noalloc(dc.key, dc.value, dc.slot_mapping, on, dc.q, kn, vn,
                                     dc.block_tables, dc.context_lens, float(case.scale),
                                     case.max_context_len, P, k_scale=dc.k_scale,
                                     v_scale=dc.v_scale)
    torch.cuda.synchronize()
    return oa, on, (ka, va, kn, vn)


@pytest.mark.parametrize("pair", PAIRS, ids=["-".join(p) for p in PAIRS])
def test_noalloc_two_calls_second_smaller(pair):
    P = 64
    for name in pair:
        case = synth.make_case(SPECS[name], 11)
        print(f"[noalloc] {name} workspace (slots, counters) "
              f"{pa.balanced_sizes(case.S, case.Hq, case.Hkv, case.D)}", flush=True)
        dc = to_device(case)
        oa, on, (ka, va, kn, vn) = step_both(case, dc, P)
        assert np.array_equal(dev_to_host(kn).view(np.uint8), dev_to_host(ka).view(np.uint8))
        assert np.array_equal(dev_to_host(vn).view(np.uint8), dev_to_host(va).view(np.uint8))
        assert np.array_equal(dev_to_host(on), dev_to_host(oa)), f"{name}: output differs"
        ok, ov = oracle.fill_cache(case)
        assert np.array_equal(dev_to_host(kn).view(np.uint8), ok.view(np.uint8))
        ref = oracle.decode_case(case, ok, ov)
        err = np.abs(as_f64(on) - ref).max()
        print(f"[noalloc] {name} max err {err:.3e}", flush=True)
        assert err <= tol(case)


@pytest.mark.timeout(600)
def test_noalloc_full_size_default_step():
    """The large mixed copy-on-write batch (256 sequences, 64 query / 8 kv
    heads, pieces of >= 128 tokens) fits the static array; output and pool are
    bit-identical to the allocating call, then a smaller batch follows."""
    for spec, seed in ((C[5], 5), (C[2], 2)):
        print(f"[noalloc] full size {spec.name}", flush=True)
        case = synth.make_case(spec, seed)
        dc = to_device(case)
        oa, on, (ka, va, kn, vn) = step_both(case, dc, 128)
        assert np.isfinite(as_f64(on)).all()
        assert np.array_equal(dev_to_host(kn).view(np.uint8), dev_to_host(ka).view(np.uint8))
        assert np.array_equal(dev_to_host(on), dev_to_host(oa)), f"{spec.name}: output differs"


def test_noalloc_refuses_shapes_beyond_the_array():
    """More (sequence, kv head) counters than the array holds: status 'shape',
    returned before any pointer is read or any kernel enqueued."""
    lib = pa._lib
    dummy = torch.zeros(16, dtype=torch.int64, device="cuda")
    p = dummy.data_ptr()
    stream = torch.cuda.current_stream().cuda_stream
    S, Hq, Hkv, D = 40000, 64, 8, 128                  # 320000 counters > 262144
    rc = lib.pa_write_decode_balanced_noalloc(p, p, p, p, p, p, p, p, 1, p, None, None,
                                              ctypes.c_float(1.0), S, Hq, Hkv, D, 32, 1, 1, 128,
                                              pa.PA_BF16, pa.PA_BF16, stream)
    assert rc == -2, pa.status_string(rc)             # PA_ERR_SHAPE
