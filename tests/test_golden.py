"""The oracle against hand-derived fixtures (tests/golden/closed_forms.json)."""
import json
import math
import os

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
with open(os.path.join(HERE, "golden", "closed_forms.json")) as fh:
    CASES = json.load(fh)["cases"]


def _num(x):
    return float("nan") if x == "nan" else float(x)


def _expr(s):
    return float(eval(s, {"__builtins__": {}}, {"e": math.e}))   # fixture strings only


def _pool(c):
    NB, Hkv, B, D = c["num_blocks"], c["num_kv_heads"], c["block_size"], c["head_dim"]
    dt = np.int8 if c["dtype"] == "i8" else np.float32
    if dt == np.int8:
        k = np.zeros((NB, Hkv, B, D), dtype=np.int8)
        v = np.zeros((NB, Hkv, B, D), dtype=np.int8)
    else:
        k = np.full((NB, Hkv, B, D), np.nan, dtype=np.float32)
        v = np.full((NB, Hkv, B, D), np.nan, dtype=np.float32)
    for s, per_head in enumerate(c["tokens"]):
        for g, toks in enumerate(per_head):
            for t, (kr, vr) in enumerate(toks):
                blk = c["block_tables"][s][t // B]
                k[blk, g, t % B] = kr
                v[blk, g, t % B] = vr
    return k, v


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_golden(case):
    assert case["citation"] and case["derivation"]
    op = case["op"]
    if op == "decode":
        k, v = _pool(case)
        q = np.array(case["q"], dtype=np.float32)
        ks = np.array(case["k_scale"], dtype=np.float32) if "k_scale" in case else None
        vs = np.array(case["v_scale"], dtype=np.float32) if "v_scale" in case else None
        got = oracle.decode(q, k, v, np.array(case["block_tables"], dtype=np.int32),
                            np.array(case["context_lens"], dtype=np.int32), case["scale"],
                            k_scale=ks, v_scale=vs)
    elif op == "reduce":
        got = oracle.splitk_reduce(np.array(case["o"]), np.array(case["m"]), np.array(case["l"]),
                                   np.array(case["context_lens"], dtype=np.int32),
                                   case["partition_size"])
    else:
        assert op == "write"
        NB, Hkv, B, D = case["num_blocks"], case["num_kv_heads"], case["block_size"], case["head_dim"]
        k = np.zeros((NB, Hkv, B, D), dtype=np.int8)
        v = np.zeros((NB, Hkv, B, D), dtype=np.int8)
        key = np.array([[[_num(x) for x in r] for r in t] for t in case["key"]], dtype=np.float32)
        val = np.array([[[_num(x) for x in r] for r in t] for t in case["value"]], dtype=np.float32)
        slots = np.array(case["slot_mapping"], dtype=np.int64)
        oracle.write_kv_cache(key, val, k, v, slots, np.array(case["k_scale"], dtype=np.float32),
                              np.array(case["v_scale"], dtype=np.float32))
        s0 = int(slots[0])
        assert k[s0 // B, 0, s0 % B].tolist() == case["expected_k_codes"]
        assert v[s0 // B, 0, s0 % B].tolist() == case["expected_v_codes"]
        return
    want = np.array([[[_expr(x) for x in row] for row in head] for head in case["expected"]])
    rtol = case.get("rtol", 0.0)
    if rtol == 0.0:
        assert np.array_equal(got, want), (got, want)
    else:
        assert np.allclose(got, want, rtol=rtol, atol=0.0), (got, want)
