"""Host model of the balanced decode schedule (``balanced_setup``, ``locate``,
``chunk_at``, ``piece_bounds``, ``next_pos`` and ``PieceEnd`` in
``csrc/pa_decode_common.hpp``), CPU only.

The model repeats the device code's integer arithmetic for a launch of W
workgroups of NWG waves and checks, for the launch shapes the GPU tests and the
bench make:

* the pieces (one per wave range; the model can also cut each range into a
  head and a tail) partition the chunk list:
  every chunk of every (sequence, kv head) segment is walked by exactly one
  piece, in list order, and every walked chunk is a chunk of its segment (its
  block-table entry lies inside the context);
* a segment wholly inside one piece is finished there; every other segment
  receives one partial from each piece that holds its chunks, in the slot
  2k (the piece's first segment, started in an earlier piece) or 2k + 1 (its
  last, going on past the piece), the slots of all pieces are distinct and
  below 4 x waves, and the piece range [first, first + pieces) that the
  combine reads is exactly the set of pieces that stored a partial, with the
  slots the combine computes for them;
* the claim flags (one per range), the workgroup done counter and the tail
  descriptors (10 int32 per range) lie inside the counters the workspace
  query reports (segment counters, then 11 per wave, then two).

At 8 query heads per kv head on a bf16 cache the 16x16 core takes pairs of
sequences per segment ("units"): the model then builds the units the way the
device does (the shared leading chunks from the block tables, capped below
both sequences' last chunks) and checks that every chunk a unit walks is a
chunk of its sequence inside its context, and every shared one a chunk that
both sequences' tables place on the same block.

A planted mistake (every partial stored in slot 2k, the first-segment slot,
so that a piece's last segment overwrites its first) is caught, and so is a
pair table that shares one chunk too many. Nothing here runs on the GPU.
"""
import math

import numpy as np
import pytest

import synth

CHUNK, CC, SC4, SC8, FAST, FAST_COW, TAIL = 16, 16, 32, 64, 160, 152, 48


class Plan:
    pass


def units_of(lens, tables, B, pair, extra_shared=0):
    """(nu, info): the chunk count of every unit and, per unit, (first
    sequence, L0, L1, n0, ns) -- the device's load_unit and
    pair_shared_chunks. tables: the block tables (rows of block ids), used
    for pair units only. extra_shared plants a mistake (one shared chunk too
    many)."""
    lens = np.asarray(lens, np.int64)
    S = len(lens)
    if not pair:
        n = (lens + CHUNK - 1) // CHUNK
        return n, [(s, int(lens[s]), 0, int(n[s]), 0) for s in range(S)]
    cpb = B // CHUNK
    nu, info = [], []
    for u in range((S + 1) // 2):
        s0 = 2 * u
        L0 = int(lens[s0])
        L1 = int(lens[s0 + 1]) if s0 + 1 < S else 0
        ns = 0
        if L0 > 0 and L1 > 0:
            cap = min((L0 - 1) // CHUNK, (L1 - 1) // CHUNK)
            if cap > 0:
                nb = -(-cap // cpb)
                run = 0
                while run < nb and tables[s0][run] == tables[s0 + 1][run]:
                    run += 1
                ns = min(cap, run * cpb)
            ns = min(ns + extra_shared, cap) if extra_shared and cap > 0 else ns
        n0 = -(-L0 // CHUNK)
        nu.append(n0 + -(-L1 // CHUNK) - ns)
        info.append((s0, L0, L1, n0, ns))
    return np.asarray(nu, np.int64), info


def setup(lens, shared_next, Hkv, G, NWG, W, P, B, tails, units=None):
    """balanced_setup: shared_next[s] is whether s and s + 1 start on the same
    physical block (both longer than a block); units: (nu, info) of
    units_of (default: one sequence per unit)."""
    S = len(lens)
    if units is None:
        units = units_of(lens, None, B, False)
    n, info = units
    U = len(n)
    SC = SC8 if G >= 8 else SC4
    K = -(-U // (NWG * 64)) if U else 0
    cost = np.where(n > 0, n * CC + SC, 0)
    cum_chunks, cum_cost = [], []
    run_n = run_c = 0
    for t in range(NWG * 64):
        ub = min(U, t * K)
        ue = min(U, ub + K)
        run_n += int(n[ub:ue].sum())
        run_c += int(cost[ub:ue].sum())
        cum_chunks.append(run_n)
        cum_cost.append(run_c)
    p = Plan()
    p.S, p.U, p.Hkv, p.K, p.sc, p.B = S, U, Hkv, K, SC, B
    p.n, p.info = n, info
    p.cum_chunks, p.cum_cost = np.array(cum_chunks, np.int64), np.array(cum_cost, np.int64)
    p.T, p.Tc = Hkv * run_n, Hkv * run_c
    p.Th, p.Tch = run_n, run_c
    p.Wv = W * NWG
    C = -(-p.Tc // p.Wv)
    cmin = max(1, P // CHUNK) * CC
    p.hm = int(np.sum(shared_next)) * 4 >= S
    if NWG == 8:
        p.H = NWG // 2
        p.Cs = max(cmin, 2 * C * (256 - (FAST_COW if p.hm else FAST)) // 256)
        p.Cf = max(p.Cs, 2 * C - p.Cs)
    else:
        p.H = 0
        p.Cs = p.Cf = max(cmin, C)

    def tail_of(ln):
        t = ln * TAIL // 256 if tails else 0
        return t if (t >= cmin and ln - t >= cmin) else 0
    p.Tf, p.Ts = tail_of(p.Cf), tail_of(p.Cs)
    if p.Tf == 0 or p.Ts == 0:
        p.Tf = p.Ts = 0
    p.PPR = 2 if p.Tf else 1
    return p


def span(p):
    return p.H * (p.Cf + p.Cs) if p.H else p.Cs


def start(p, j):
    if not p.H:
        return j * p.Cs
    w, v = divmod(j, 2 * p.H)
    return w * span(p) + (v * p.Cf if v < p.H else p.H * p.Cf + (v - p.H) * p.Cs)


def range_of(p, X):
    if not p.H:
        return X // p.Cs
    w, o = divmod(X, span(p))
    return w * 2 * p.H + (o // p.Cf if o < p.H * p.Cf else p.H + (o - p.H * p.Cf) // p.Cs)


def fast(p, j):
    return p.H and (j % (2 * p.H)) < p.H


def rlen(p, j):
    return p.Cf if fast(p, j) else p.Cs


def tail(p, j):
    return p.Tf if fast(p, j) else p.Ts


def pstart(p, k):
    if p.PPR == 1:
        return start(p, k)
    j = k >> 1
    return start(p, j) + ((rlen(p, j) - tail(p, j)) if (k & 1) else 0)


def piece_of(p, X):
    j = range_of(p, X)
    if p.PPR == 1:
        return j
    return 2 * j + (1 if X >= start(p, j) + rlen(p, j) - tail(p, j) else 0)


def locate(p, Y):
    g, Yt, mul = 0, Y, p.Hkv
    if p.hm:
        g = Y // p.Tch
        Yt = Y - g * p.Tch
        mul = 1
    t = int(np.sum(mul * p.cum_cost <= Yt))
    assert t < len(p.cum_cost), "locate: past the last slice"
    base = int(p.cum_chunks[t - 1]) * mul if t else 0
    cbase = int(p.cum_cost[t - 1]) * mul if t else 0
    if p.hm:
        base += g * p.Th
        cbase += g * p.Tch
    ub = min(p.U, t * p.K)
    ue = min(p.U, ub + p.K)
    found = None
    for u in range(ub, ue):
        nn = int(p.n[u])
        c = mul * (nn * CC + p.sc) if nn else 0
        if Y < cbase + c:
            found = u
            break
        base += mul * nn
        cbase += c
    assert found is not None, "locate: position not in its slice"
    return found, int(p.n[found]), g, base, cbase


def chunk_at(p, Y):
    """(list index, SegPos dict or None)."""
    if Y >= p.Tc:
        return p.T, None
    s, nn, g0, base, cbase = locate(p, Y)
    sc = nn * CC + p.sc
    g = g0 if p.hm else (Y - cbase) // sc
    gb = 0 if p.hm else g
    off = (Y - cbase) - gb * sc
    assert 0 <= off < sc
    c = 0 if off < p.sc else (off - p.sc) // CC
    pos = dict(s=s, n=nn, g=g, c=c, A=base + gb * nn, Y=cbase + gb * sc + p.sc)
    return base + gb * nn + c, pos


def chunk_ref(p, q):
    """(sequence, its chunk, its length, columns 0 all / 1 first / 2 second,
    shared) of chunk q["c"] of unit q["s"] (the device's chunk_ref)."""
    s0, L0, L1, n0, ns = p.info[q["s"]]
    c = q["c"]
    if c < ns:
        return s0, c, L0, 0, True
    if c < n0:
        return s0, c, L0, 1, False
    return s0 + 1, c - n0 + ns, L1, 2, False


def next_pos(p, q):
    q = dict(q)
    if q["c"] + 1 < q["n"]:
        q["c"] += 1
        return q
    q["c"] = 0
    q["Y"] += q["n"] * CC + p.sc
    q["A"] += q["n"]
    if p.hm:
        while True:
            q["s"] += 1
            if q["s"] == p.U:
                q["s"] = 0
                q["g"] += 1
            assert q["g"] < p.Hkv, "next_pos: walked past the last head"
            q["n"] = int(p.n[q["s"]])
            if q["n"]:
                return q
    q["g"] += 1
    if q["g"] < p.Hkv:
        return q
    q["g"] = 0
    while True:
        q["s"] += 1
        assert q["s"] < p.U, "next_pos: walked past the last unit"
        q["n"] = int(p.n[q["s"]])
        if q["n"]:
            return q


def chunk_list(p):
    """(u, g, c) of every list index, in list order."""
    out = []
    order = ([(g, u) for g in range(p.Hkv) for u in range(p.U)] if p.hm else
             [(g, u) for u in range(p.U) for g in range(p.Hkv)])
    for g, u in order:
        for c in range(int(p.n[u])):
            out.append((u, g, c))
    return out


def simulate(lens, shared_next, Hkv, G, NWG, W, P, B, tails, planted=False, tables=None,
             pair=False, extra_shared=0):
    lens = np.asarray(lens, np.int64)
    units = units_of(lens, tables, B, pair, extra_shared)
    p = setup(lens, shared_next, Hkv, G, NWG, W, P, B, tails, units)
    want = chunk_list(p)
    assert len(want) == p.T
    owner = np.full(p.T, -1, np.int64)
    stored = {}                                        # (segment) -> {piece: slot}
    finals = set()
    slots = set()
    declared = {}                                      # segment -> (first, pieces)
    for k in range(p.PPR * p.Wv):
        Y0 = pstart(p, k)
        if Y0 >= p.Tc:
            continue
        X0, cur = chunk_at(p, Y0)
        X1, _ = chunk_at(p, min(p.Tc, pstart(p, k + 1)))
        if X0 >= X1:
            continue
        q = cur
        for i in range(X1 - X0):
            X = X0 + i
            assert owner[X] < 0, f"chunk {X} walked twice"
            owner[X] = k
            assert want[X] == (q["s"], q["g"], q["c"]), f"chunk {X}: {want[X]} vs walk"
            sq, cc, Lq, who, sh_ = chunk_ref(p, q)
            assert sq < p.S and (cc * CHUNK) // B < -(-Lq // B), "block-table entry past the context"
            if sh_:                                    # a shared chunk: full, and on one block for both
                assert (cc + 1) * CHUNK < Lq and (cc + 1) * CHUNK < lens[sq + 1], "shared chunk not full"
                assert tables[sq][cc * CHUNK // B] == tables[sq + 1][cc * CHUNK // B], \
                    "shared chunk on different blocks"
            assert q["A"] + q["c"] == X
            last = i + 1 == X1 - X0
            if last or q["c"] + 1 == q["n"]:           # a segment end inside the piece
                seg = (q["s"], q["g"])
                Bn = q["A"] + q["n"]
                if q["A"] >= X0 and Bn <= X1:
                    finals.add(seg)
                else:
                    first = piece_of(p, q["Y"] + CC - 1)
                    pieces = piece_of(p, q["Y"] + q["n"] * CC - 1) - first + 1
                    slot = 2 * k + (1 if q["A"] >= X0 and not planted else 0)
                    assert slot not in slots, f"slot {slot} stored twice"
                    assert slot < 2 * p.PPR * p.Wv
                    slots.add(slot)
                    stored.setdefault(seg, {})[k] = slot
                    assert declared.setdefault(seg, (first, pieces)) == (first, pieces)
            if not last:
                q = next_pos(p, q)
    assert (owner >= 0).all(), "a chunk no piece walks"
    for seg, ks in stored.items():
        assert seg not in finals
        first, pieces = declared[seg]
        assert sorted(ks) == list(range(first, first + pieces)), f"segment {seg}: pieces"
        for i in range(pieces):
            assert ks[first + i] == 2 * (first + i) + (1 if i == 0 else 0), "combine slot"
    nseg = sum(p.Hkv for u in range(p.U) if p.n[u])
    assert len(finals) + len(stored) == nseg, "a segment is neither finished nor combined"
    # claims: flags[0, Wv), the done counter and 10 int32 of descriptor per
    # range after the segment counters, inside S Hkv + 11 waves + 2 counters
    assert p.S * p.Hkv + p.Wv + 1 + 10 * p.Wv <= p.S * p.Hkv + 11 * p.Wv + 2
    return p


def shared_first_blocks(spec, lens):
    """Whether s and s + 1 start on the same physical block: with copy-on-write
    prefix groups, two sequences of one group that are both longer than a block
    share their first prefix block (synth's pool)."""
    S = len(lens)
    out = np.zeros(S, bool)
    if spec.prefix_groups:
        gsz = S // spec.prefix_groups
        for s in range(S - 1):
            out[s] = (s // gsz == (s + 1) // gsz and lens[s] > spec.block_size
                      and lens[s + 1] > spec.block_size)
    return out


def block_tables(spec, lens):
    """Block tables with synth's sharing: the sequences of a prefix group hold
    the group's blocks for their first min(prefix blocks, (L - 1) // B) logical
    blocks, every other block is their own (ids are distinct otherwise)."""
    S, B = len(lens), spec.block_size
    nxt = [0]

    def fresh():
        nxt[0] += 1
        return nxt[0]
    gsz = S // spec.prefix_groups if spec.prefix_groups else 0
    pblk = spec.prefix_tokens // B if spec.prefix_groups else 0
    groups = {}
    rows = []
    for s in range(S):
        nb = -(-int(lens[s]) // B)
        sh = min(pblk, (int(lens[s]) - 1) // B) if gsz else 0
        ids = groups.setdefault(s // gsz, [fresh() for _ in range(pblk)]) if gsz else []
        rows.append(list(ids[:sh]) + [fresh() for _ in range(nb - sh)] + [0])
    return rows


def pairs_used(spec):
    """The balanced kernel takes pair units: the 16x16 core (8 query heads per
    kv head, head_dim 128, bf16 queries and cache) and at most 4096 sequences."""
    G = spec.num_heads // spec.num_kv_heads
    return (G == 8 and spec.head_dim == 128 and spec.act == "bf16" and spec.cache == "bf16"
            and (spec.num_seqs + 1) // 2 <= 2048)


def _cases():
    C = synth.CONFIGS
    S_ = synth.Spec
    small = {
        "cfg1": C[1], "cfg2s": C[2].replace(num_seqs=12, lens=("uniform", 1, 1100), max_len=1100),
        "cfg3s": C[3].replace(num_seqs=2, lens=("const", 4099), max_len=4099),
        "cfg4s": C[4].replace(num_seqs=10, lens=("uniform", 1, 1300), max_len=1300),
        "cfg5s": C[5].replace(num_seqs=16, lens=("lognormal", 200, 1.0, 1, 1500), max_len=1500,
                              prefix_groups=2, prefix_tokens=256),
        "g8_i8": S_("G=8 int8", 6, ("uniform", 1, 900), 32, 4, 128, 16, cache="i8", max_len=900),
        "mid_g4": S_("mid", 24, ("uniform", 1000, 3000), 32, 8, 128, 16, max_len=3000),
        "mid_g8_cow": S_("mid cow", 48, ("lognormal", 800, 1.0, 1, 6000), 64, 8, 128, 32,
                         max_len=6000, prefix_groups=4, prefix_tokens=512),
        "g2": S_("G=2", 6, ("uniform", 1, 600), 8, 4, 128, 32, max_len=600),
        "g8_odd": S_("G=8 odd", 7, ("uniform", 1, 700), 64, 8, 128, 16, max_len=700,
                     prefix_groups=1, prefix_tokens=256),
    }
    out = []
    for name, spec in small.items():
        L = synth.draw_lens(spec, 7)
        G = spec.num_heads // spec.num_kv_heads
        NWG = 8 if G in (4, 8) and spec.head_dim == 128 and spec.act == "bf16" else 4
        Ws = (256,) if NWG == 8 else (256, 512, 1024)
        for P in (16, 64, 128, 256):
            for W in Ws:
                out.append((f"{name}-P{P}-W{W}", L, spec, NWG, W, P))
        Lz = L.copy()
        Lz[[0, len(L) // 2, len(L) - 1]] = 0
        out.append((f"{name}-zeros", Lz, spec, NWG, Ws[0], 16))
    for cfg in (2, 3, 4, 5):
        spec = C[cfg]
        L = synth.draw_lens(spec, cfg)
        out.append((f"cfg{cfg}-P128", L, spec, 8, 256, 128))
    for n in (4096, 4097):                             # the pair table full, and one past it
        spec = S_(f"G=8 bf16 {n}", n, ("uniform", 1, 48), 64, 8, 128, 16, max_len=48,
                  prefix_groups=64 if n == 4096 else 17, prefix_tokens=16)
        out.append((f"many{n}-P128", synth.draw_lens(spec, 5), spec, 8, 256, 128))
    # odd grids (not a multiple of 8: no XCD remap) and tiny batches
    spec = C[2].replace(num_seqs=5, lens=("uniform", 1, 300), max_len=300)
    out.append(("odd-grid", synth.draw_lens(spec, 3), spec, 8, 100, 16))
    out.append(("one-seq", np.array([1], np.int32), spec.replace(num_seqs=1), 8, 256, 16))
    return out


CASES = _cases()


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_balanced_schedule(case):
    name, L, spec, NWG, W, P = case
    G = spec.num_heads // spec.num_kv_heads
    sh = shared_first_blocks(spec, L)
    pair = pairs_used(spec)
    simulate(L, sh, spec.num_kv_heads, G, NWG, W, P, spec.block_size, tails=False,
             tables=block_tables(spec, L) if pair else None, pair=pair)


def test_block_tables_follow_synth():
    """The model's tables share exactly the blocks synth's pool shares."""
    spec = synth.CONFIGS[5].replace(num_seqs=16, lens=("lognormal", 200, 1.0, 1, 1500),
                                    max_len=1500, prefix_groups=2, prefix_tokens=256)
    case = synth.make_case(spec, 11)
    L = case.context_lens
    mine = block_tables(spec, L)
    for a in range(len(L)):
        for b in range(len(L)):
            for lb in range(-(-int(min(L[a], L[b])) // spec.block_size)):
                assert ((case.block_tables[a][lb] == case.block_tables[b][lb])
                        == (mine[a][lb] == mine[b][lb])), (a, b, lb)


def test_pair_units_of_the_cow_batch():
    """The mixed copy-on-write batch as pair units: most pairs share their
    prefix chunks, and the walk covers every chunk once."""
    spec = synth.CONFIGS[5]
    L = synth.draw_lens(spec, 5)
    tab = block_tables(spec, L)
    nu, info = units_of(L, tab, spec.block_size, True)
    shared = sum(i[4] for i in info)
    assert shared * CHUNK > 0.4 * (412020 - 223252) / 2
    assert int(nu.sum()) + shared == int(((np.asarray(L) + CHUNK - 1) // CHUNK).sum())


def test_planted_pair_table_mistake_is_caught():
    spec = synth.CONFIGS[5].replace(num_seqs=16, lens=("lognormal", 200, 1.0, 1, 1500),
                                    max_len=1500, prefix_groups=2, prefix_tokens=256)
    L = synth.draw_lens(spec, 7)
    with pytest.raises(AssertionError):
        simulate(L, shared_first_blocks(spec, L), 8, 8, 8, 256, 16, spec.block_size,
                 tails=False, tables=block_tables(spec, L), pair=True, extra_shared=1)


def test_cow_batch_is_head_major():
    spec = synth.CONFIGS[5]
    L = synth.draw_lens(spec, 5)
    p = setup(L, shared_first_blocks(spec, L), 8, 8, 8, 256, 128, 32, False)
    assert p.hm and p.PPR == 1


def test_planted_slot_mistake_is_caught():
    spec = synth.CONFIGS[4]
    L = synth.draw_lens(spec, 4)
    with pytest.raises(AssertionError):
        simulate(L, np.zeros(len(L), bool), 8, 4, 8, 256, 128, 16, tails=False, planted=True)


def test_head_tail_cut_partitions_too():
    """The head / tail cut of every range (two pieces per range) also partitions
    the list with the same slot rule (a variant of the schedule that was built,
    measured and not kept)."""
    spec = synth.CONFIGS[4]
    L = synth.draw_lens(spec, 4)
    p = simulate(L, np.zeros(len(L), bool), 8, 4, 8, 256, 128, 16, tails=True)
    assert p.PPR == 2


def test_all_empty():
    spec = synth.CONFIGS[2]
    p = simulate(np.zeros(8, np.int64), np.zeros(8, bool), 8, 4, 8, 256, 64, 16, tails=False)
    assert p.T == 0
