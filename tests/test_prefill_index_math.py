"""Host model of the multi-query kernel's grid mapping and address arithmetic
(``prefill_kernel`` in ``csrc/pa_prefill.hip``), CPU only.

For every launch shape the GPU tests and the bench use, the model walks every
workgroup, wave, lane and KV tile of the launch exactly as the kernel indexes
them -- the workgroup -> (row tile, kv head, sequence, partition) map with the
XCD-contiguous order and the placement by length, the tile loop with its
block ids fetched one tile ahead, the per-piece load addresses, the new-token
rows of the fused write, the query loads and the output / partial stores --
and checks that every index lies inside the buffer it addresses:

* block-table entries read are among the ``ceil(L / B)`` entries of the
  sequence's context;
* every K/V load stays inside its (block, kv head) tile of the pool;
* every row read from ``key`` / ``value`` (fused write) or ``q``, and every
  row written to ``out`` or the split-K workspace, is a row of the call.

It also plants, in a copy of the model, the indexing mistake that made the
fused write read past ``key`` / ``value`` (spare waves of the last iteration,
whose tiles lie wholly past the context, taking a new-token row at
``jn >= n``) and checks the model flags it, so the check would have caught it.
Nothing here runs on the GPU.
"""
import numpy as np
import pytest

import synth

PD, TK = 128, 32


def launch_shape(max_query_len, G):
    """(NR, MB, row tiles) as launch_prefill picks them."""
    rows = max_query_len * G
    if rows <= 16:
        return 1, 1, 1
    if rows <= 64:
        return 2, 2, 1
    return 4, 2, (rows + 127) // 128


def snake_seq(lens, p, pair=True):
    """Sequence taking place p of the XCD-contiguous list (snake_place); pair:
    every workgroup resident at once, the run's second half reversed."""
    S = len(lens)
    per = S // 8
    x, j0 = p // per, p % per
    half = per // 2
    j = j0 if (not pair or j0 < half) else per - 1 - (j0 - half)
    r = 8 * j + (7 - x if j & 1 else x)
    order = sorted(range(S), key=lambda t: (-int(lens[t]), t))   # rank r -> sequence
    return order[r]


def _piece_tables():
    """Token row t and first element e of every thread's piece k of a tile,
    per (NR, int8): piece p = ti + k TPT is token p / PPR, elements
    (p % PPR) EPP .., with ti = rg 64 + lane (all 256 threads; waves of one
    token group cover ti = 0 .. TPT - 1, the others repeat them)."""
    T_, E_ = {}, {}
    tid = np.arange(256)
    for NR in (1, 2, 4):
        for i8 in (False, True):
            TPT, EPP = NR * 64, 16 if i8 else 8
            PPR = PD // EPP
            NLD = TK * PPR // TPT
            ti = ((tid >> 6) % NR) * 64 + (tid & 63)
            T_[(NR, i8)] = [(ti + k * TPT) // PPR for k in range(NLD)]
            E_[(NR, i8)] = [((ti + k * TPT) % PPR) * EPP for k in range(NLD)]
    return T_, E_


PIECE_T, PIECE_E = _piece_tables()


class OOB(AssertionError):
    pass


def check(cond, what):
    if not np.all(cond):
        raise OOB(what)


def model_launch(lens, qlens, Hq, Hkv, B, i8=False, wr=False, P=0, max_query_len=None,
                 planted_jn_bound=False, planted_masked_half=False):
    """Walk one launch; raise OOB at the first out-of-range index. Returns the
    number of workgroups that did work (a sanity count)."""
    lens = np.asarray(lens, np.int64)
    qlens = np.asarray(qlens, np.int64)
    S = len(lens)
    G = Hq // Hkv
    qsl = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int64)
    T = int(qsl[-1])
    mq = int(qlens.max()) if max_query_len is None else max_query_len
    maxL = int(lens.max())
    NR, MB, row_tiles = launch_shape(mq, G)
    NT = 4 // NR
    RT = NR * MB * 16
    TPT = NR * 64
    EPP = 16 if i8 else 8
    PPR = PD // EPP
    NLD = TK * PPR // TPT
    ELT = 1 if i8 else 2
    TILE_BYTES = B * PD * ELT
    TOK_PER_LD = TPT // PPR
    HALF_UNIFORM = TOK_PER_LD <= 16
    NP = -(-maxL // P) if P else 1
    W = row_tiles * NP * Hkv * S
    spread = row_tiles == 1 and NP > 1
    snake = row_tiles == 1 and NP == 1 and W % 8 == 0 and S % 8 == 0 and S <= 256

    tid = np.arange(256)
    lane, wave = tid & 63, tid >> 6
    rg = wave % NR
    col = lane & 15
    busy = 0
    for w0 in range(W):
        w = w0 if (W % 8 or spread) else (w0 % 8) * (W // 8) + w0 // 8
        rt, rest = w % row_tiles, w // row_tiles
        sg = rest // NP
        part = (rest + sg) % NP if spread else rest % NP
        g = sg % Hkv
        # one round on MI355X: two workgroups per CU for these instances, 256 CUs
        s = snake_seq(lens, sg // Hkv, pair=W <= 512) if snake else sg // Hkv
        check(0 <= s < S, "sequence index")
        q0, n, L = int(qsl[s]), int(qlens[s]), int(lens[s])
        tiles = (n * G + RT - 1) // RT
        if rt >= tiles:
            continue
        tile = tiles - 1 - rt
        TQ = RT // G
        tok0 = tile * TQ
        p_first = L - n + tok0
        limit = p_first + min(TQ, n - tok0)
        t_begin = part * P if P else 0
        if t_begin >= limit:
            continue
        busy += 1
        kt0 = t_begin // TK
        nkt = (min(limit, t_begin + P) + TK - 1) // TK if P else (limit + TK - 1) // TK
        nit = (nkt - kt0 + NT - 1) // NT
        new0 = L - n
        nvalid = (L + B - 1) // B                      # block-table entries of the context

        if wr:                                         # prologue: the tile's new tokens
            ntok = min(TQ, n - tok0)
            idx = np.arange(ntok * (PD // 8))
            j = tok0 + idx // (PD // 8)
            pos = new0 + j
            keep = (pos >= t_begin) & (pos < t_begin + P) if P else np.ones_like(j, bool)
            check(q0 + j[keep] < T, "fused write: key/value row")

        for mb in range(MB):                           # query rows
            r = (rg * MB + mb) * 16 + col
            j, h = r // G, r % G
            valid = tok0 + j < n
            check(q0 + tok0 + j[valid] < T, "q row")
            check(g * G + h < Hq, "query head")
            if P:
                slot = ((q0 + tok0 + j[valid]) * Hq + g * G + h[valid]) * NP + part
                check(slot < T * Hq * NP, "split-K slot")
                check(part < NP, "partition")

        # every KV tile any wave of the workgroup loads: wave tg loads tiles
        # kt0 + it NT + tg for it < nit (the spares of the last iteration
        # included), each with the block ids tile_bases fetched for that same
        # tile (fetched one tile ahead into bnext, which is overwritten only
        # after the load that uses it has been issued). With two register
        # tiles in flight (a tile of at most 2 pieces per thread and pool) the
        # loads are unconditional: tiles it < nit + 2 are loaded and the block
        # ids of it < nit + 3 fetched.
        depth = 2 if NLD <= 2 else 1
        n_load = nit + 2 if depth == 2 else nit
        n_bases = nit + 3 if depth == 2 else nit
        kts = (kt0 + np.arange(n_load)[:, None] * NT + np.arange(NT)[None, :]).reshape(-1)
        kbs = (kt0 + np.arange(n_bases)[:, None] * NT + np.arange(NT)[None, :]).reshape(-1)
        for hf in range(2):                            # tile_bases, every tile asked for
            T0 = kbs * TK + 16 * hf
            check(T0[T0 < limit] // B < nvalid, "block-table entry past the context")
        fetched = []
        for hf in range(2):                            # the bases each loaded tile uses
            T0 = kts * TK + 16 * hf
            f = T0 < limit
            fetched.append(f)
        if wr:                                         # load_tile: the tile's new-token slots
            j0 = kts * TK - new0
            has = (j0 + TK > 0) & (j0 < n)
            for jj in j0[has]:
                tb, te = max(0, -int(jj)), min(TK, n - int(jj))
                check(q0 + jj + tb >= 0 and q0 + jj + te - 1 < T, "slot_mapping entry")
            if i8:                                     # the new tokens' scales, per half
                for hf in range(2):
                    T0 = kts[has] * TK + 16 * hf
                    check(T0[T0 < limit] // B < nvalid, "new-token scale's block")
        for k in range(NLD):                           # load_tile
            t, e = PIECE_T[(NR, i8)][k], PIECE_E[(NR, i8)][k]
            inn = kts[:, None] * TK + t[None, :] < limit
            lo = (np.where(inn, (t % B)[None, :], 0) * PD + e[None, :]) * ELT
            check(lo + 16 <= TILE_BYTES, "piece inside its (block, kv head) tile")
            if HALF_UNIFORM:
                half = np.broadcast_to(np.full_like(t, (k * TOK_PER_LD) // 16)[None, :], inn.shape)
            else:
                half = np.broadcast_to((t >= 16).astype(np.int64)[None, :], inn.shape)
            for hv in (0, 1):
                need = inn & (half == hv)
                check(~need | fetched[hv][:, None], "piece of a block never fetched")
            # a piece past the context reads token 0 of its half's base, which
            # must be a block of the context whenever the tile is computed (the
            # masked weight is 0, but 0 times a non-finite pool value is not):
            # half 1 wholly past the context takes half 0's base
            live = kts < nkt
            for hv in (0, 1):
                own = fetched[hv] if hv == 0 else (fetched[1] | fetched[0])
                past = ~inn & (half == hv) & live[:, None]
                check(~past | own[:, None], "masked piece read outside the context")
            if wr:
                jn = kts[:, None] * TK + np.where(inn, t[None, :], 0) - new0
                sel = (jn >= 0) if planted_jn_bound else (jn >= 0) & (jn < n)
                check((q0 + jn[sel] < T) & (q0 + jn[sel] >= 0),
                      "new-token row read from key/value")
                # Which position each piece of a computed tile reads from the
                # cache: none where it comes from key / value (a tile holding
                # new tokens, jn a new token); else its own token, or, past
                # `limit`, the first token of the block of its base -- base 0
                # in a tile holding new tokens, its half's base elsewhere.
                # None may be a new token (the launch writes those slots while
                # it reads: another workgroup's, or its own without a barrier).
                j0 = kts * TK - new0
                fresh = ((j0 + TK > 0) & (j0 < n))[:, None]
                from_key = fresh & (jn >= 0) & (jn < n)
                blk0 = np.where(kts * TK < limit, kts * TK, -1)[:, None]
                hb = kts[:, None] * TK + 16 * half
                blkh = np.where(hb < limit, hb // B * B, blk0)
                blk = np.where(fresh & ~np.asarray(planted_masked_half), blk0, blkh)
                pos = np.where(inn, kts[:, None] * TK + t[None, :], blk)
                live_p = (kts < nkt)[:, None]
                check(~(live_p & ~from_key & (pos >= new0) & (pos < new0 + n)),
                      "cache read of a new token the launch writes")
                # a piece of EPP cache elements reads EPP bf16 activations
                check(e + EPP <= PD, "new-token piece inside its key/value row")
        if i8:                                         # compute: int8 scales
            live = kts[kts < nkt]
            for tt in range(2):
                T0 = live * TK + tt * 16
                check(T0[T0 < limit] // B < nvalid, "int8 scale's block")
    return busy


# ---- launch shapes used by the GPU tests and the bench -----------------------

def _cases():
    C = synth.CONFIGS
    S_ = synth.Spec
    out = []
    # tests/test_gpu_prefill.py CASES (seed 11, query counts from seed 12)
    tests = {
        "verify_g4": (C[2].replace(num_seqs=12, lens=("uniform", 1, 1100), max_len=1100),
                      ("const", 4)),
        "verify_g4_i8": (C[4].replace(num_seqs=10, lens=("uniform", 1, 1300), max_len=1300),
                         ("const", 4)),
        "verify_g8_b32": (S_("G=8 B=32", 8, ("uniform", 1, 900), 32, 4, 128, 32, max_len=900),
                          ("uniform", 1, 8)),
        "g2_i8_b32": (S_("G=2 int8 B=32", 6, ("uniform", 1, 700), 8, 4, 128, 32, cache="i8",
                         max_len=700), ("uniform", 0, 20)),
        "g16": (S_("G=16", 5, ("uniform", 1, 600), 16, 1, 128, 16, max_len=600),
                ("uniform", 1, 3)),
        "mixed_g4": (S_("G=4 mixed", 9, ("uniform", 1, 800), 16, 4, 128, 16, max_len=800),
                     ("uniform", 0, 40)),
        "chunk_g4": (S_("chunk", 2, ("const", 1500), 8, 2, 128, 16, max_len=1500),
                     ("const", 300)),
        "chunk_i8_g8": (S_("chunk i8", 2, ("uniform", 600, 1000), 16, 2, 128, 32, cache="i8",
                           max_len=1000), ("const", 100)),
        "whole_mha": (S_("whole", 3, ("uniform", 1, 200), 4, 4, 128, 16, max_len=200), "whole"),
        "cow_g8": (C[5].replace(num_seqs=16, lens=("lognormal", 200, 1.0, 1, 1500),
                                max_len=1500, prefix_groups=2, prefix_tokens=256),
                   ("uniform", 1, 5)),
        "decode_ties_s64": (C[2].replace(num_seqs=64, lens=("uniform", 1, 40), max_len=40),
                            ("const", 1)),
        "decode_s256": (C[2].replace(num_seqs=256, lens=("uniform", 1, 300), max_len=300),
                        ("const", 1)),
        "decode_s264": (C[2].replace(num_seqs=264, lens=("uniform", 1, 300), max_len=300),
                        ("const", 1)),
    }
    # (name, P, fused write): the calls tests/test_gpu_prefill.py makes
    used = [(nm, 0, False) for nm in tests] + [
        ("verify_g4", 64, False), ("verify_g4_i8", 512, False), ("verify_g8_b32", 32, False),
        ("g2_i8_b32", 96, False), ("mixed_g4", 128, False), ("chunk_g4", 256, False),
        ("whole_mha", 32, False), ("cow_g8", 512, False),
        ("verify_g4", 0, True), ("verify_g8_b32", 0, True), ("mixed_g4", 0, True),
        ("chunk_g4", 0, True), ("whole_mha", 0, True), ("cow_g8", 0, True),
        ("decode_ties_s64", 0, True), ("decode_s256", 0, True), ("verify_g4", 64, True),
        ("chunk_g4", 256, True), ("cow_g8", 512, True), ("verify_g4_i8", 0, True),
        ("g2_i8_b32", 0, True), ("chunk_i8_g8", 0, True), ("verify_g4_i8", 64, True),
        ("chunk_i8_g8", 256, True)]
    for name, P, wr in used:
        spec, ql = tests[name]
        if name == "cow_g8" and wr:
            ql = ("const", 1)                          # one new token per sequence there
        L = synth.draw_lens(spec, 11)
        if ql == "whole":
            n = L.astype(np.int64)
        else:
            n = synth.query_counts(L, ql, np.random.default_rng(12))
        out.append((f"{name}-P{P}" + ("-write" if wr else ""), L, n, spec,
                    spec.cache == "i8", wr, P))
    # the bench's multi-query steps: one row per sequence on the bf16 and
    # int8 workloads, the new tokens written by the same launch, split or
    # not; the verify and prefill workloads
    for cfg, P in ((2, 0), (3, 2048), (3, 4096), (4, 0), (5, 1024)):
        spec = C[cfg]
        L = synth.draw_lens(spec, cfg)
        n = np.ones(len(L), np.int64)
        out.append((f"cfg{cfg}-P{P}-write", L, n, spec, spec.cache == "i8", True, P))
    for name in ("verify", "verify_long", "prefill"):
        spec, ql = synth.MULTI_QUERY[name]
        L = synth.draw_lens(spec, 2)
        n = synth.query_counts(L, ql, np.random.default_rng(3))
        for P in ((spec.partition_size, 4096) if name == "verify_long" else (0,)):
            out.append((f"{name}-P{P}", L, n, spec, False, False, P))
    return out


CASES = _cases()


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_prefill_launch_in_bounds(case):
    name, L, n, spec, i8, wr, P = case
    if spec.num_heads // spec.num_kv_heads > 16 or 16 % (spec.num_heads // spec.num_kv_heads):
        pytest.skip("group size not covered by the kernel")
    if int(n.sum()) == 0:
        pytest.skip("no query rows: nothing is launched")
    busy = model_launch(L, n, spec.num_heads, spec.num_kv_heads, spec.block_size, i8=i8, wr=wr,
                        P=P)
    assert busy > 0


def test_planted_jn_bound_is_caught():
    """The fused write's mistake that faulted on the GPU -- spare waves of the
    last iteration reading a new-token row at jn >= n -- is an out-of-range
    read in the model."""
    spec = synth.CONFIGS[2].replace(num_seqs=64, lens=("uniform", 1, 40), max_len=40)
    L = synth.draw_lens(spec, 11)
    n = np.ones(len(L), np.int64)
    with pytest.raises(OOB, match="new-token row"):
        model_launch(L, n, spec.num_heads, spec.num_kv_heads, spec.block_size, wr=True,
                     planted_jn_bound=True)
    model_launch(L, n, spec.num_heads, spec.num_kv_heads, spec.block_size, wr=True)


@pytest.mark.parametrize("name", ["mixed_g4", "decode_b16", "decode_b16_i8"])
def test_planted_masked_half_base_is_caught(name):
    """Masked pieces (past the tile's last row) of a tile holding new tokens
    read the first token of their half's block: with 16-token blocks that
    token may be a new one, whose slot the same launch is writing -- the NaN
    poison of a new token's slot then reached an output through a zero
    weight. The model flags it; taking base 0 (the tile's first token: an
    older token, or a new one read from key / value) does not. decode: one
    new token per sequence at the first position of a tile's second half
    (L = 32 k + 17)."""
    if name.startswith("decode"):
        L = np.array([17, 49, 81, 113, 145, 177, 209, 1041], np.int64)
        n = np.ones(len(L), np.int64)
        Hq, Hkv, B, i8 = 32, 8, 16, name.endswith("i8")
    else:
        cases = {c[0]: c for c in CASES}
        _, L, n, spec, i8, wr, P = cases[f"{name}-P0-write"]
        Hq, Hkv, B = spec.num_heads, spec.num_kv_heads, spec.block_size
    with pytest.raises(OOB, match="new token the launch writes"):
        model_launch(L, n, Hq, Hkv, B, i8=i8, wr=True, planted_masked_half=True)
    model_launch(L, n, Hq, Hkv, B, i8=i8, wr=True)


def test_snake_place_is_a_permutation():
    """Every sequence gets exactly one place (ties in length broken by index)."""
    rng = np.random.default_rng(0)
    for S in (8, 40, 64, 72, 256):
        lens = rng.integers(1, 40, size=S)
        for pair in (False, True):
            got = sorted(snake_seq(lens, p, pair) for p in range(S))
            assert got == list(range(S))
