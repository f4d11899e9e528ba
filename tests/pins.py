"""Pins of the fp64 oracle against things other than itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError
(or the oracle's own error) when the oracle disagrees with what the
mathematics fixes. They are run as ordinary tests (test_oracle_pins.py) and
against deliberately broken builds of the oracle (test_oracle_mutants.py),
which must each fail at least one pin.

What pins what:
* un-paging: the paged result over the oracle-written pool equals dense
  attention computed by torch's scaled_dot_product_attention in float64 on
  the *source* K/V tensors (never written into a pool) -- pins the write, the
  block-table gather, GQA head mapping, the scale, the softmax and PV;
* brute force: 40-digit ``decimal`` attention on tiny inputs (its ``exp`` is
  correctly rounded), over block sizes 1..4, head dims 1..3, groups 1..3;
* closed forms: L = 1 returns V exactly; constant V = 2^k returns it exactly;
  q = 0 or scale = 0 gives the mean of V; two tokens give the sigmoid mix;
* one-hot probe: a logit that dominates by > 745 returns its V row exactly;
* placement: renaming physical blocks, or un-sharing copy-on-write prefixes,
  leaves the output bit-identical;
* split-K: each partition's (o, m, l) equals dense attention over that token
  range and logsumexp; the reduce equals a logsumexp-weighted mix;
* int8 write: every code equals exact-rational rounding (fp32 quotient with
  ties to even, then integer with ties to even, clamp to +-127);
* several query tokens per sequence: torch SDPA over the dense source K/V with
  an explicit causal mask aligned to the end of the context, and, row by row,
  one-token decode over the context cut after the row's position.
"""
from __future__ import annotations

import dataclasses
import math
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import torch

import oracle
import synth

# --------------------------------------------------------------------------
# helpers (harness side: un-paging from source tensors)
# --------------------------------------------------------------------------


def source_rows(case):
    """Map each physical slot to its source token row in concat([pre, new])."""
    NB, B = case.num_blocks, case.B
    idx = np.full(NB * B, -1, dtype=np.int64)
    idx[case.pre_slots] = np.arange(len(case.pre_slots))
    idx[case.slot_mapping] = len(case.pre_slots) + np.arange(len(case.slot_mapping))
    kall = np.concatenate([case.pre_key, case.key])
    vall = np.concatenate([case.pre_value, case.value])
    return idx, kall, vall


def dense_kv(case, k_pool=None, v_pool=None):
    """Per sequence, dense float64 K and V [L, Hkv, D] in logical order.

    Float caches: taken from the source token values. int8 caches: the codes
    in the given pool times their (block, kv head) scale."""
    B = case.B
    out = []
    if case.spec.cache == "i8":
        for s in range(case.S):
            L = int(case.context_lens[s])
            p = np.arange(L)
            b = case.block_tables[s, p // B].astype(np.int64)
            o = p % B
            k = k_pool[b, :, o, :].astype(np.float64) * case.k_scale[b][:, :, None].astype(np.float64)
            v = v_pool[b, :, o, :].astype(np.float64) * case.v_scale[b][:, :, None].astype(np.float64)
            out.append((k, v))
        return out
    idx, kall, vall = source_rows(case)
    k64 = synth.as_f32(kall, case.spec.act).astype(np.float64)
    v64 = synth.as_f32(vall, case.spec.act).astype(np.float64)
    for s in range(case.S):
        L = int(case.context_lens[s])
        p = np.arange(L)
        slots = case.block_tables[s, p // B].astype(np.int64) * B + p % B
        rows = idx[slots]
        assert (rows >= 0).all(), "in-context slot never written"
        out.append((k64[rows], v64[rows]))
    return out


def q64(case):
    return synth.as_f32(case.q, case.spec.act).astype(np.float64)


def sdpa_ref(qs, k, v, scale):
    """torch SDPA, float64 CPU: qs [Hq, D], k/v [L, Hkv, D] -> [Hq, D]."""
    Hq, D = qs.shape
    Hkv = k.shape[1]
    qt = torch.from_numpy(qs).reshape(1, Hq, 1, D)
    kt = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2))).reshape(1, Hkv, -1, D)
    vt = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2))).reshape(1, Hkv, -1, D)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=float(scale),
                                                         enable_gqa=(Hq != Hkv))
    return o.reshape(Hq, D).numpy()


def small_specs():
    """Small workloads spanning the dtypes, GQA groups, block sizes and a
    copy-on-write prefix."""
    return [
        synth.CONFIGS[1],
        synth.Spec("gqa bf16", 5, ("uniform", 1, 70), 8, 2, 32, 16, act="bf16", cache="bf16",
                   max_len=70),
        synth.Spec("gqa int8", 4, ("uniform", 1, 50), 6, 2, 16, 8, act="bf16", cache="i8",
                   max_len=50),
        synth.Spec("int8 fp32 act", 3, ("uniform", 5, 40), 2, 2, 8, 4, act="f32", cache="i8",
                   max_len=40),
        synth.Spec("cow prefix", 8, ("uniform", 2, 60), 4, 1, 16, 4, act="f32", cache="f32",
                   max_len=60, prefix_groups=2, prefix_tokens=16),
        synth.Spec("B32 G8", 3, ("uniform", 20, 90), 16, 2, 32, 32, act="bf16", cache="bf16",
                   max_len=96),
    ]


# --------------------------------------------------------------------------
# pins
# --------------------------------------------------------------------------


def pin_unpaged_sdpa(ora, seeds=(0, 1)):
    for spec in small_specs():
        for seed in seeds:
            case = synth.make_case(spec, seed)
            k, v = ora.fill_cache(case)
            got = ora.decode_case(case, k, v)
            dense = dense_kv(case, k, v)
            qq = q64(case)
            for s in range(case.S):
                ref = sdpa_ref(qq[s], *dense[s], case.scale)
                err = np.abs(got[s] - ref).max()
                assert err <= 1e-12, f"{spec.name} seed {seed} seq {s}: |oracle - sdpa| = {err}"


def _decimal_attention(qs, k, v, scale, G):
    """40-digit attention: qs [Hq, D], k/v [L, Hkv, D] (floats) -> [Hq, D]."""
    getcontext().prec = 40
    Hq, D = qs.shape
    L = k.shape[0]
    sc = Decimal(float(scale))
    out = np.empty((Hq, D))
    for h in range(Hq):
        g = h // G
        qd = [Decimal(float(x)) for x in qs[h]]
        x = [sc * sum(qd[d] * Decimal(float(k[t, g, d])) for d in range(D)) for t in range(L)]
        M = max(x)
        w = [(xi - M).exp() for xi in x]
        Z = sum(w)
        for d in range(D):
            out[h, d] = float(sum(w[t] * Decimal(float(v[t, g, d])) for t in range(L)) / Z)
    return out


def pin_decimal_bruteforce(ora, n_cases=40, seed=1234):
    rng = np.random.default_rng(seed)
    for i in range(n_cases):
        B = int(rng.choice([1, 2, 4]))
        D = int(rng.integers(1, 4))
        G = int(rng.integers(1, 4))
        Hkv = int(rng.integers(1, 3))
        S = 2
        lens = tuple(int(x) for x in rng.integers(1, 3 * B + 2, size=S))
        spec = synth.Spec(f"bf{i}", S, ("fixed", lens), G * Hkv, Hkv, D, B, act="f32",
                          cache="f32", max_len=3 * B + 1, pool=("factor", 2.0))
        case = synth.make_case(spec, 100 + i)
        k, v = ora.fill_cache(case)
        got = ora.decode_case(case, k, v)
        dense = dense_kv(case)
        qq = q64(case)
        for s in range(S):
            ref = _decimal_attention(qq[s], *dense[s], case.scale, G)
            err = np.abs(got[s] - ref).max()
            assert err <= 1e-13, f"brute force case {i} seq {s}: err {err}"


def _with_values(case, kfun=None, vfun=None, qfun=None):
    """Copy of ``case`` with K/V/Q replaced (float32 activations only)."""
    import dataclasses
    assert case.spec.act == "f32"
    new = dataclasses.replace(case)
    if kfun:
        new.pre_key, new.key = kfun(case.pre_key.copy()), kfun(case.key.copy())
    if vfun:
        new.pre_value, new.value = vfun(case.pre_value.copy()), vfun(case.value.copy())
    if qfun:
        new.q = qfun(case.q.copy())
    return new


def pin_closed_forms(ora):
    # L = 1: the only token's V, exactly (fp32 and bf16, MHA and GQA)
    for spec in (synth.Spec("L1 f32", 6, ("const", 1), 4, 2, 16, 16, act="f32", cache="f32",
                            max_len=16),
                 synth.Spec("L1 bf16", 6, ("const", 1), 8, 2, 32, 16, act="bf16", cache="bf16",
                            max_len=16)):
        case = synth.make_case(spec, 3)
        got = ora.decode_case(case)
        v = synth.as_f32(case.value, spec.act).astype(np.float64)      # [S, Hkv, D]
        G = spec.group_size
        want = np.repeat(v, G, axis=1)
        assert np.array_equal(got, want), "L = 1 must return V exactly"

    base = synth.Spec("cf", 5, ("uniform", 1, 45), 6, 3, 8, 4, act="f32", cache="f32", max_len=45)
    case = synth.make_case(base, 4)
    # constant V = 2^k: exactly that constant
    for c in (0.25, 4.0, -2.0):
        cc = _with_values(case, vfun=lambda a, c=c: np.full_like(a, c))
        got = ora.decode_case(cc)
        assert np.array_equal(got, np.full_like(got, c)), f"constant V = {c} not returned exactly"
    # q = 0 and scale = 0: the mean of V over the context
    dense = dense_kv(case)
    for variant in ("q0", "scale0"):
        if variant == "q0":
            cc = _with_values(case, qfun=np.zeros_like)
        else:
            import dataclasses
            cc = dataclasses.replace(case, scale=np.float32(0.0))
        got = ora.decode_case(cc)
        for s in range(case.S):
            vmean = np.array([[math.fsum(dense[s][1][:, h // 2, d]) / case.context_lens[s]
                               for d in range(case.D)] for h in range(case.Hq)])
            err = np.abs(got[s] - vmean).max()
            assert err <= 1e-14, f"{variant}: mean of V mismatch {err}"
    # two tokens: sigmoid mix
    two = synth.Spec("two", 4, ("const", 2), 4, 2, 8, 4, act="f32", cache="f32", max_len=2)
    case = synth.make_case(two, 5)
    got = ora.decode_case(case)
    dense = dense_kv(case)
    qq = q64(case)
    for s in range(case.S):
        k, v = dense[s]
        for h in range(case.Hq):
            g = h // 2
            x0 = float(case.scale) * math.fsum(qq[s, h] * k[0, g])
            x1 = float(case.scale) * math.fsum(qq[s, h] * k[1, g])
            s1 = 1.0 / (1.0 + math.exp(x0 - x1))
            s0 = 1.0 / (1.0 + math.exp(x1 - x0))
            want = s1 * v[1, g] + s0 * v[0, g]
            err = np.abs(got[s, h] - want).max()
            assert err <= 1e-14, f"two-token closed form err {err}"


def pin_onehot(ora):
    """q = 128 e_0, k_{t*} = 128 e_0 and every other k_0 = 0 make logit t*
    exceed all others by 128 * 128 * scale = 2048, so every other weight
    exp(-2048) is exactly 0 in fp64 and the output is v_{t*} bit for bit."""
    spec = synth.CONFIGS[1]
    case = synth.make_case(spec, 1)
    maxL = int(case.context_lens.max())
    idx, _, _ = source_rows(case)
    B = case.B
    for tstar in range(maxL):
        ts = [tstar % int(L) for L in case.context_lens]

        def kf(a):
            a[:, :, 0] = 0.0
            return a
        cc = _with_values(case, kfun=kf, qfun=lambda a: np.zeros_like(a))
        cc.q[:, :, 0] = 128.0
        # raise k_0 of token t*_s in each sequence (through its source row)
        npre = len(case.pre_slots)
        for s, t in enumerate(ts):
            slot = int(case.block_tables[s, t // B]) * B + t % B
            r = idx[slot]
            if r < npre:
                cc.pre_key[r, :, 0] = 128.0
            else:
                cc.key[r - npre, :, 0] = 128.0
        got = ora.decode_case(cc)
        dense = dense_kv(cc)
        for s, t in enumerate(ts):
            want = np.repeat(dense[s][1][t], case.Hq // case.Hkv, axis=0)   # [Hq, D]
            assert np.array_equal(got[s], want), f"one-hot t*={t} seq {s} not exact"


def pin_placement(ora):
    for spec, seed in ((synth.CONFIGS[1], 9), (small_specs()[1], 2), (small_specs()[4], 3),
                       (small_specs()[2], 4)):
        case = synth.make_case(spec, seed)
        ref = ora.decode_case(case)
        for ps in (11, 12):
            got = ora.decode_case(synth.permute_placement(case, ps))
            assert np.array_equal(got, ref), f"{spec.name}: block permutation changed the output"
        if spec.prefix_groups:
            got = ora.decode_case(synth.unshare_prefixes(case))
            assert np.array_equal(got, ref), "un-sharing CoW prefixes changed the output"


def pin_splitk(ora):
    for spec, P in ((small_specs()[1], 16), (small_specs()[5], 32), (synth.CONFIGS[1], 16),
                    (small_specs()[2], 8)):
        case = synth.make_case(spec, 6)
        k, v = ora.fill_cache(case)
        o, m, l = ora.decode_partials(case.q, k, v, case.block_tables, case.context_lens,
                                      case.scale, P, case.k_scale, case.v_scale)
        dense = dense_kv(case, k, v)
        qq = q64(case)
        G = spec.group_size
        for s in range(case.S):
            L = int(case.context_lens[s])
            kd, vd = dense[s]
            for j in range(-(-L // P)):
                t0, t1 = j * P, min(L, (j + 1) * P)
                ref = sdpa_ref(qq[s], kd[t0:t1], vd[t0:t1], case.scale)
                assert np.abs(o[s, :, j] - ref).max() <= 1e-12, "partition output mismatch"
                kt = torch.from_numpy(np.repeat(kd[t0:t1], G, axis=1).transpose(1, 0, 2).copy())
                x = torch.einsum("hd,htd->ht", torch.from_numpy(qq[s]), kt) * float(case.scale)
                mx = x.max(dim=1).values.numpy()
                lse = torch.logsumexp(x, dim=1).numpy()
                assert np.abs(m[s, :, j] - mx).max() <= 1e-12, "partition max mismatch"
                assert np.abs(np.log(l[s, :, j]) + m[s, :, j] - lse).max() <= 1e-12, \
                    "partition sum mismatch"
            # partitions past the length are never written
            assert np.isnan(o[s, :, -(-L // P):]).all()
        full = ora.decode_case(case, k, v)
        red = ora.splitk_reduce(o, m, l, case.context_lens, P)
        assert np.abs(red - full).max() <= 1e-12, "reduce(partials) != single pass"
        # P >= L: one partition, whose output is the single-pass output
        Pbig = -(-int(case.context_lens.max()) // case.B) * case.B
        o1, m1, l1 = ora.decode_partials(case.q, k, v, case.block_tables, case.context_lens,
                                         case.scale, Pbig, case.k_scale, case.v_scale)
        assert o1.shape[2] == 1 and np.array_equal(o1[:, :, 0], full)
    # the reduce alone against a logsumexp-weighted mix of random partials
    rng = np.random.default_rng(7)
    S, H, NP, D, P = 3, 4, 5, 6, 16
    lens = np.array([1, 40, 80], dtype=np.int32)
    o = rng.standard_normal((S, H, NP, D))
    m = rng.standard_normal((S, H, NP)) * 30
    l = rng.uniform(0.5, 20, (S, H, NP))
    got = ora.splitk_reduce(o, m, l, lens, P)
    for s in range(S):
        n = -(-int(lens[s]) // P)
        a = torch.from_numpy(m[s, :, :n] + np.log(l[s, :, :n]))
        w = torch.softmax(a, dim=1).numpy()
        want = np.einsum("hj,hjd->hd", w, o[s, :, :n])
        assert np.abs(got[s] - want).max() <= 1e-12, "reduce mismatch"


# ---- int8 write ---------------------------------------------------------------

def _round_rational_to_f32(fr: Fraction) -> Fraction:
    """Exact round-to-nearest-even of a rational to binary32 (no overflow case
    needed here: |values| stay far below 2^128)."""
    if fr == 0:
        return Fraction(0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    # 2^e <= a < 2^(e+1)
    e = max(e, -126)
    quantum = Fraction(2) ** (e - 23)
    n = a / quantum
    fl = n.numerator // n.denominator
    r = n - fl
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * quantum


def _rint_even(fr: Fraction) -> int:
    fl = fr.numerator // fr.denominator
    r = fr - fl
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return int(fl)


def expected_code(x: float, s: float) -> int:
    if math.isnan(x):
        return 0
    if math.isinf(x):
        return 127 if (x > 0) == (s > 0) else -127
    q = _round_rational_to_f32(Fraction(x) / Fraction(s))
    r = _rint_even(q)
    return max(-127, min(127, r))


def near_tie_pairs(n_scales=3000, seed=31, limit=64):
    """(x, s) pairs, x a bf16 value and s an fp32 scale, whose exact quotient
    is not a half-integer but lies within half an fp32 ulp of one, so the
    correctly rounded fp32 quotient *is* the half-integer. Rounding the exact
    (or fp64) quotient to an integer gives the other neighbour here."""
    rng = np.random.default_rng(seed)
    vals = synth.bf16_to_f32(np.arange(65536, dtype=np.uint32).astype(np.uint16))
    fin = vals[np.isfinite(vals) & (vals != 0)]
    out = []
    for sc in rng.uniform(1e-3, 1e-1, n_scales).astype(np.float32):
        x = fin[np.abs(fin) <= 127 * float(sc)]
        qv = x.astype(np.float64) / float(sc)
        frac = qv - np.floor(qv)
        cand = np.nonzero((np.abs(frac - 0.5) < 2.0 ** -18) & (frac != 0.5))[0]
        for i in cand:
            fr = Fraction(float(x[i])) / Fraction(float(sc))
            f32q = _round_rational_to_f32(fr)
            if f32q.denominator == 2 and fr != f32q:
                out.append((np.float32(x[i]), sc))
        if len(out) >= limit:
            break
    return out


def pin_write_int8(ora, per_scale=1500, seed=21):
    # near ties: one (block, head) per pair, each with its own scale
    pairs = near_tie_pairs()
    assert len(pairs) >= 8, "near-tie search found too few cases"
    n = len(pairs)
    key = synth.bf16_bits(np.array([p[0] for p in pairs], dtype=np.float32)).reshape(n, 1, 1)
    k = np.full((n, 1, 1, 1), -128, dtype=np.int8)
    v = k.copy()
    ks = np.array([p[1] for p in pairs], dtype=np.float32).reshape(n, 1)
    ora.write_kv_cache(key, key.copy(), k, v, np.arange(n, dtype=np.int64), ks, ks)
    want = np.array([expected_code(float(x), float(s)) for x, s in pairs], dtype=np.int8)
    assert np.array_equal(k.reshape(-1), want), "near-tie int8 codes wrong"

    rng = np.random.default_rng(seed)
    scales = [np.float32(1 / 127), np.float32(0.0123), np.float32(3.7e-3), np.float32(1.0),
              np.float32(2.0 ** -3), np.float32(5.3e-5)]
    all_bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = synth.bf16_to_f32(all_bits)
    D = 64
    for sc in scales:
        near = np.nonzero(np.abs(vals) <= 130 * float(sc))[0]
        far = np.nonzero(~(np.abs(vals) <= 130 * float(sc)))[0]
        pick = np.concatenate([
            rng.choice(near, size=min(per_scale, near.size), replace=False),
            rng.choice(far, size=200, replace=False),
        ])
        if sc == np.float32(2.0 ** -3):
            # exact ties k + 1/2 for every k in [-128, 127]
            ties = synth.bf16_bits(((np.arange(-128, 128) + 0.5) / 8).astype(np.float32))
            pick = np.concatenate([pick, ties.astype(np.int64)])
        bits = all_bits[pick]
        T = -(-bits.size // D)
        pad = np.zeros(T * D - bits.size, dtype=np.uint16)
        key = np.concatenate([bits, pad]).reshape(T, 1, D)
        value = key[::-1].copy()
        NB = T + 1
        k = np.full((NB, 1, 1, D), -128, dtype=np.int8)
        v = k.copy()
        ks = np.full((NB, 1), sc, dtype=np.float32)
        slots = np.arange(T, dtype=np.int64)
        ora.write_kv_cache(key, value, k, v, slots, ks, ks)
        xs = synth.bf16_to_f32(key.reshape(-1))
        want = np.array([expected_code(float(x), float(sc)) for x in xs], dtype=np.int8)
        assert np.array_equal(k[:T].reshape(-1), want), f"int8 key codes wrong at scale {sc}"
        xv = synth.bf16_to_f32(value.reshape(-1))
        wantv = np.array([expected_code(float(x), float(sc)) for x in xv], dtype=np.int8)
        assert np.array_equal(v[:T].reshape(-1), wantv), f"int8 value codes wrong at scale {sc}"
        assert (k[T] == -128).all(), "write touched an unwritten block"
        finite = np.isfinite(xs) & (np.abs(xs) <= 127 * float(sc))
        err = np.abs(xs[finite].astype(np.float64) - want[finite] * float(sc))
        assert (err <= float(sc) / 2 * (1 + 1e-6)).all(), "|x - q s| > s/2"


def pin_write_copy(ora):
    rng = np.random.default_rng(22)
    for act in ("f32", "bf16"):
        NB, Hkv, B, D, T = 9, 3, 4, 8, 20
        k32 = rng.standard_normal((T, Hkv, D)).astype(np.float32)
        v32 = rng.standard_normal((T, Hkv, D)).astype(np.float32)
        key = synth.bf16_bits(k32) if act == "bf16" else k32
        value = synth.bf16_bits(v32) if act == "bf16" else v32
        slots = rng.permutation(NB * B)[:T].astype(np.int64)
        slots[::5] = -1                               # skipped tokens
        dt = np.uint16 if act == "bf16" else np.uint32
        poison = 0x7FC0 if act == "bf16" else 0x7FC00000
        k = np.full((NB, Hkv, B, D), poison, dtype=dt)
        v = k.copy()
        kv = k.view(np.float32) if act == "f32" else k
        vv = v.view(np.float32) if act == "f32" else v
        ora.write_kv_cache(key, value, kv, vv, slots)
        kb = key.view(dt)
        vb = value.view(dt)
        written = np.zeros((NB, B), dtype=bool)
        for i, sl in enumerate(slots):
            if sl < 0:
                continue
            b, o = divmod(int(sl), B)
            assert np.array_equal(k[b, :, o, :], kb[i]), "key bits not copied"
            assert np.array_equal(v[b, :, o, :], vb[i]), "value bits not copied"
            written[b, o] = True
        untouched = ~written
        assert (k.transpose(0, 2, 1, 3)[untouched] == poison).all(), "stray key write"
        assert (v.transpose(0, 2, 1, 3)[untouched] == poison).all(), "stray value write"


def pin_zero_length(ora):
    case = synth.make_case(synth.CONFIGS[1], 1)
    k, v = ora.fill_cache(case)
    lens = case.context_lens.copy()
    lens[2] = 0
    got = ora.decode(case.q, k, v, case.block_tables, lens, case.scale)
    assert np.array_equal(got[2], np.zeros_like(got[2])), "L = 0 must give zeros"
    assert np.isfinite(got).all()


def pin_copy_blocks(ora):
    """Copy-on-write copy: a sequence that gets private copies of its shared
    prefix blocks (its table repointed at the copies) attends to the same values,
    so the oracle's decode must be bit-identical -- whatever the copy drops (V,
    a kv head, the int8 scales) or misplaces changes it. Every byte outside the
    destination blocks is untouched, and invalid mappings are refused."""
    cow = synth.Spec("cow prefix, 2 kv heads", 8, ("uniform", 2, 60), 4, 2, 16, 4, act="bf16",
                     cache="bf16", max_len=60, prefix_groups=2, prefix_tokens=16)
    for spec, seed in ((cow, 3), (cow.replace(cache="i8"), 5), (small_specs()[4], 4)):
        case = synth.make_case(spec, seed)
        k, v = ora.fill_cache(case)
        ref = ora.decode_case(case, k, v)
        B = case.B
        nblk = -(-case.context_lens.astype(np.int64) // B)
        used = set(int(b) for s in range(case.S) for b in case.block_tables[s, :nblk[s]])
        free = [b for b in range(case.num_blocks) if b not in used and b != case.poison_block]
        pairs, bt = [], case.block_tables.copy()
        for s in range(case.S):
            for lb in range(int(nblk[s])):
                b = int(bt[s, lb])
                if case.refcount[b] > 1 and free and len(pairs) < 24:
                    dst = free.pop()
                    pairs.append((b, dst))
                    bt[s, lb] = dst
                    break
        assert len(pairs) >= 4, "the case must have shared blocks and free ones"
        k2, v2 = k.copy(), v.copy()
        ks2 = None if case.k_scale is None else case.k_scale.copy()
        vs2 = None if case.v_scale is None else case.v_scale.copy()
        ora.copy_blocks(k2, v2, np.array(pairs), ks2, vs2)
        moved = dataclasses.replace(case, block_tables=bt, k_scale=ks2, v_scale=vs2)
        got = ora.decode_case(moved, k2, v2)
        assert np.array_equal(got, ref), f"{spec.name}: decode changed after the copy"
        dsts = [d for _, d in pairs]
        keep = np.ones(case.num_blocks, dtype=bool)
        keep[dsts] = False
        assert np.array_equal(k2[keep].view(np.uint8), k[keep].view(np.uint8)), "stray K bytes"
        assert np.array_equal(v2[keep].view(np.uint8), v[keep].view(np.uint8)), "stray V bytes"
        src0, dst0 = pairs[0]
        for bad in ([(src0, dst0), (pairs[1][0], dst0)],          # one destination twice
                    [(src0, dst0), (dst0, pairs[1][1])],          # a destination is also a source
                    [(src0, case.num_blocks)], [(src0, src0)]):    # out of range; onto itself
            try:
                ora.copy_blocks(k2.copy(), v2.copy(), np.array(bad), ks2, vs2)
            except oracle.OracleError:
                continue
            raise AssertionError(f"invalid mapping {bad} accepted")


def _query_mixes(case, seed):
    """Query counts per sequence: a few tokens each, and each whole context."""
    return [synth.make_queries(case, ("uniform", 0, 6), seed),
            synth.make_queries(case, case.context_lens.astype(np.int64), seed + 1)]


def pin_prefill_causal_sdpa(ora, seeds=(0, 1)):
    """Several query tokens per sequence against torch SDPA (float64) over the
    dense source K/V with an explicit mask: query j of n at position L - n + j
    sees tokens 0 .. L - n + j."""
    for spec in small_specs():
        for seed in seeds:
            case = synth.make_case(spec, seed)
            k, v = ora.fill_cache(case)
            dense = dense_kv(case, k, v)
            for qs in _query_mixes(case, 10 * seed):
                got = ora.prefill(qs.q, k, v, case.block_tables, case.context_lens,
                                  qs.query_start_loc, case.scale, case.k_scale, case.v_scale)
                q = synth.as_f32(qs.q, spec.act).astype(np.float64)
                for s in range(case.S):
                    a, b = int(qs.query_start_loc[s]), int(qs.query_start_loc[s + 1])
                    n, L = b - a, int(case.context_lens[s])
                    if n == 0:
                        continue
                    kk, vv = dense[s]
                    Hq, D, Hkv = case.Hq, case.D, case.Hkv
                    qt = torch.from_numpy(np.ascontiguousarray(q[a:b].transpose(1, 0, 2)))
                    kt = torch.from_numpy(np.ascontiguousarray(kk.transpose(1, 0, 2)))
                    vt = torch.from_numpy(np.ascontiguousarray(vv.transpose(1, 0, 2)))
                    pos = L - n + np.arange(n)
                    mask = torch.from_numpy(np.arange(L)[None, :] <= pos[:, None])
                    ref = torch.nn.functional.scaled_dot_product_attention(
                        qt[None], kt[None], vt[None], attn_mask=mask, scale=float(case.scale),
                        enable_gqa=(Hq != Hkv))[0].numpy().transpose(1, 0, 2)
                    err = np.abs(got[a:b] - ref).max()
                    assert err <= 1e-12, f"{spec.name} seed {seed} seq {s}: |oracle - sdpa| = {err}"


def pin_prefill_rows_are_decode(ora):
    """Row j of sequence s equals one-token decode of that query over the
    context truncated after its position (the decode oracle is pinned by the
    pins above)."""
    for spec in small_specs()[:4]:
        case = synth.make_case(spec, 3)
        k, v = ora.fill_cache(case)
        for qs in _query_mixes(case, 7):
            got = ora.prefill(qs.q, k, v, case.block_tables, case.context_lens,
                              qs.query_start_loc, case.scale, case.k_scale, case.v_scale)
            seq = np.repeat(np.arange(case.S), qs.q_lens)
            j = np.arange(qs.num_tokens) - qs.query_start_loc[seq]
            pos = case.context_lens[seq] - qs.q_lens[seq] + j
            ref = ora.decode(qs.q, k, v, case.block_tables[seq], (pos + 1).astype(np.int32),
                             case.scale, case.k_scale, case.v_scale)
            assert np.array_equal(got, ref), f"{spec.name}: prefill rows differ from decode"


ALL_PINS = [pin_unpaged_sdpa, pin_decimal_bruteforce, pin_closed_forms, pin_onehot,
            pin_placement, pin_splitk, pin_write_int8, pin_write_copy, pin_zero_length,
            pin_copy_blocks, pin_prefill_causal_sdpa, pin_prefill_rows_are_decode]
