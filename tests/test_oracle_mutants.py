"""Planted mistakes in the oracle must each fail at least one pin.

Each mutant is a copy of oracle/oracle.c with one plausible mistake (a dropped
term, a wrong sign, a wrong or transposed index, the wrong rounding), built
with gcc into a temporary directory and run through every pin in a child
process (a mutant may read out of bounds; the child keeps that away from the
test runner). A mutant that passes every pin means the pins have a blind spot.
"""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

# (name, text to find, replacement)
MUTANTS = [
    ("drop the scale", "return p->scale * acc;", "return acc;"),
    ("exp sign flipped", "double w = exp(x[t - t0] - M);", "double w = exp(M - x[t - t0]);"),
    ("GQA head map modulo", "int64_t g = h / (p->Hq / p->Hkv);\n    int64_t o",
     "int64_t g = h % p->Hkv;\n    int64_t o"),
    ("token offset off by one", "int64_t o = t % p->B;", "int64_t o = (t + 1) % p->B;"),
    ("cache index transposed", "return ((b * p->Hkv + g) * p->B + o) * p->D + d;",
     "return ((b * p->Hkv + g) * p->D + d) * p->B + o;"),
    ("kv head index swapped with block", "return ((b * p->Hkv + g) * p->B + o) * p->D + d;",
     "return ((g * p->NB + b) * p->B + o) * p->D + d;"),
    ("no normalisation", "o_out[d] /= Z;", "o_out[d] /= 1.0;"),
    ("last token dropped", "attend_range(&p, s, s, h, 0, L, o, &m, &l, x)",
     "attend_range(&p, s, s, h, 0, L > 1 ? L - 1 : L, o, &m, &l, x)"),
    ("prefill drops the diagonal", "attend_range(&p, s, r, h, 0, pos + 1,",
     "attend_range(&p, s, r, h, 0, pos > 0 ? pos : 1,"),
    ("prefill sees one token ahead", "attend_range(&p, s, r, h, 0, pos + 1,",
     "attend_range(&p, s, r, h, 0, pos + 1 < context_lens[s] ? pos + 2 : pos + 1,"),
    ("prefill rows counted from the front",
     "int64_t pos = context_lens[s] - n + (r - query_start_loc[s]);",
     "int64_t pos = r - query_start_loc[s];"),
    ("prefill reads the sequence's first query row", "attend_range(&p, s, r, h, 0, pos + 1,",
     "attend_range(&p, s, query_start_loc[s], h, 0, pos + 1,"),
    ("prefill row to sequence off by one", "while (query_start_loc[s + 1] <= r)",
     "while (query_start_loc[s + 1] < r)"),
    ("dequant scale dropped", "x *= (double)sc[b * p->Hkv + g];", "x *= 1.0;"),
    ("int8 truncation", "float r = nearbyintf(t);", "float r = truncf(t);"),
    ("int8 ties away from zero", "float r = nearbyintf(t);", "float r = roundf(t);"),
    ("int8 range -128", "if (r < -127.0f)\n        r = -127.0f;", "if (r < -128.0f)\n        r = -128.0f;"),
    ("int8 rounds the fp64 quotient", "float r = nearbyintf(t);",
     "float r = (float)nearbyint(x / (double)s);"),
    ("reduce weight sign", "double W = l_part[sh * NP + j] * exp(m_part[sh * NP + j] - M);",
     "double W = l_part[sh * NP + j] * exp(M - m_part[sh * NP + j]);"),
    ("reduce drops the sums", "double W = l_part[sh * NP + j] * exp(m_part[sh * NP + j] - M);",
     "double W = exp(m_part[sh * NP + j] - M);"),
    ("partition end not clipped", "int64_t t1 = (j + 1) * P < L ? (j + 1) * P : L;",
     "int64_t t1 = (j + 1) * P;"),
    ("write ignores skip", "if (slot < 0)\n            continue;\n        int64_t b",
     "if (slot < -1)\n            continue;\n        int64_t b"),
    ("copy drops V",
     "memcpy((char *)v_cache + dst * bytes, (const char *)v_cache + src * bytes, (size_t)bytes);",
     ";"),
    ("copy moves one kv head",
     "const int64_t bytes = (int64_t)num_kv_heads * block_size * head_dim * elem_size(cache_dtype);",
     "const int64_t bytes = (int64_t)block_size * head_dim * elem_size(cache_dtype);"),
    ("copy keeps the destination's scales",
     "k_scale[dst * num_kv_heads + g] = k_scale[src * num_kv_heads + g];", ";"),
    ("copy direction swapped",
     "int64_t src = block_mapping[2 * i], dst = block_mapping[2 * i + 1];\n        memcpy",
     "int64_t dst = block_mapping[2 * i], src = block_mapping[2 * i + 1];\n        memcpy"),
]

CHILD = r"""
import sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import oracle, pins
ora = oracle.Oracle({lib!r})
for pin in pins.ALL_PINS:
    try:
        pin(ora)
    except Exception as e:
        print("caught by", pin.__name__, ":", type(e).__name__, str(e)[:120])
        sys.exit(1)
print("NOT CAUGHT")
sys.exit(0)
"""


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new, tmp_path):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name!r} not found"
    mutant = src.replace(old, new, 1)
    csrc = tmp_path / "oracle_mutant.c"
    csrc.write_text(mutant)
    lib = tmp_path / "liboracle_mutant.so"
    sys.path.insert(0, os.path.join(ROOT, "oracle"))
    import build as obuild
    sys.path.pop(0)
    flags = [f for f in obuild.FLAGS if f != "-Werror"]
    subprocess.run(["gcc", *flags, str(csrc), "-o", str(lib), "-lm"], check=True)
    code = CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=str(lib))
    env = dict(os.environ, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                       timeout=600)
    assert "NOT CAUGHT" not in r.stdout, f"mutant {name!r} passed every pin"
    assert r.returncode != 0, f"mutant {name!r}: child exited 0\n{r.stdout}\n{r.stderr}"
