"""Seeded synthetic decode batches for paged-attention decode.

This module is shared input plumbing: both the fp64 oracle (under ``oracle/``)
and the HIP path consume what it makes. It holds none of the method's
arithmetic -- no dot products, softmax, quantisation or cache writes. It only:

* draws context lengths, Q and the K/V values of every in-context token;
* rounds fp32 draws to bf16 bit patterns (the workloads' activation dtype);
* runs a host-side block pool (free list + refcounts) that hands out shuffled
  physical block ids, including copy-on-write shared prefixes, and builds the
  per-sequence logical->physical ``block_tables`` and the ``slot_mapping`` of
  every token to be written;
* chooses the caller-side int8 scales (absmax/127 per (block, kv head)).

The cache itself is *not* filled here: each side (oracle, HIP) fills its own
pool by running its own slot-mapped write over ``pre_*`` (the tokens already in
context) and then ``key``/``value`` (the one new token per sequence).

Paging model: "Paged KV-cache -- fixed-size physical block pool with a
per-sequence logical->physical page table, copy-on-write reference counting"
(Continuous-Batching-LLM-Inference-Engine README, feature list).
"""
from __future__ import annotations

import collections
import dataclasses
import math
from typing import Optional

import numpy as np

ACT_DTYPES = ("f32", "bf16")
CACHE_DTYPES = ("f32", "bf16", "i8")

# Poison patterns written into every slot that no sequence has in context.
F32_POISON = np.uint32(0x7FC00000)   # quiet NaN
BF16_POISON = np.uint16(0x7FC0)      # quiet NaN
I8_POISON = np.int8(-128)            # never produced by the symmetric quantiser


# --------------------------------------------------------------------------
# bf16 bit helpers (input casting only)
# --------------------------------------------------------------------------

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 values (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def as_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    """Activation array in its storage form -> fp32 values (exact)."""
    return bf16_to_f32(x) if dtype == "bf16" else np.asarray(x, dtype=np.float32)


def storage_dtype(dtype: str):
    return {"f32": np.float32, "bf16": np.uint16, "i8": np.int8}[dtype]


def elt_bytes(dtype: str) -> int:
    return {"f32": 4, "bf16": 2, "i8": 1}[dtype]


# --------------------------------------------------------------------------
# Workload specifications
# --------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Spec:
    """Shape and distribution of one synthetic decode batch.

    ``lens`` is one of
      ("fixed", (L0, L1, ...)), ("const", L), ("uniform", lo, hi) (inclusive),
      ("lognormal", median, sigma, lo, hi) (rounded to nearest, then clipped).
    ``pool`` is ("fixed", NB) or ("factor", f): ceil(f * blocks needed) + 1
    poison block.
    """
    name: str
    num_seqs: int
    lens: tuple
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    act: str = "bf16"
    cache: str = "bf16"
    max_len: int = 0               # bound on context length -> block-table width
    pool: tuple = ("factor", 1.25)
    q_std: float = 1.0
    prefix_groups: int = 0         # >0: consecutive groups of sequences share a CoW prefix
    prefix_tokens: int = 0
    partition_size: int = 0        # split-K partition used by the workload (0 = one pass)

    @property
    def group_size(self) -> int:
        return self.num_heads // self.num_kv_heads

    @property
    def max_blocks_per_seq(self) -> int:
        return -(-self.max_len // self.block_size)

    def replace(self, **kw) -> "Spec":
        return dataclasses.replace(self, **kw)


# The five workloads of the paged decode benchmark (one GPU each).
CONFIGS = {
    1: Spec("tiny fp32 MHA", 4, ("fixed", (1, 17, 64, 100)), 4, 4, 64, 16,
            act="f32", cache="f32", max_len=100, pool=("fixed", 64)),
    2: Spec("Llama-3-8B-shaped bf16 GQA batch", 64, ("uniform", 128, 2048), 32, 8, 128, 16,
            act="bf16", cache="bf16", max_len=2048, partition_size=512),
    3: Spec("long-context split-K bf16", 8, ("const", 32768), 32, 8, 128, 16,
            act="bf16", cache="bf16", max_len=32768, q_std=2.0, partition_size=512),
    4: Spec("int8 KV cache", 128, ("uniform", 256, 4096), 32, 8, 128, 16,
            act="bf16", cache="i8", max_len=4096, partition_size=512),
    5: Spec("large mixed batch with shared prefixes", 256, ("lognormal", 1024, 1.0, 16, 16384),
            64, 8, 128, 32, act="bf16", cache="bf16", max_len=16384,
            prefix_groups=4, prefix_tokens=1024, partition_size=512),
}


# --------------------------------------------------------------------------
# Host block pool (allocation policy only)
# --------------------------------------------------------------------------

class PoolExhausted(RuntimeError):
    pass


class BlockPool:
    """Fixed pool of physical blocks with a shuffled free list and refcounts.

    Block ``poison`` (the last id) is never handed out; block-table padding
    points at it so a stray read sees poison instead of faulting.
    """

    def __init__(self, num_blocks: int, rng: np.random.Generator):
        if num_blocks < 2:
            raise ValueError("pool needs at least one usable block and the poison block")
        self.num_blocks = num_blocks
        self.poison = num_blocks - 1
        self.free = collections.deque(int(b) for b in rng.permutation(num_blocks - 1))
        self.refcount = np.zeros(num_blocks, dtype=np.int32)

    def alloc(self) -> int:
        if not self.free:
            raise PoolExhausted("block pool exhausted")
        b = self.free.popleft()
        self.refcount[b] = 1
        return b

    def share(self, b: int) -> int:
        if self.refcount[b] <= 0:
            raise ValueError(f"share of free block {b}")
        self.refcount[b] += 1
        return b

    def release(self, b: int) -> None:
        if self.refcount[b] <= 0:
            raise ValueError(f"refcount underflow on block {b}")
        self.refcount[b] -= 1
        if self.refcount[b] == 0:
            self.free.append(b)

    @property
    def num_free(self) -> int:
        return len(self.free)


# --------------------------------------------------------------------------
# A decode batch
# --------------------------------------------------------------------------

@dataclasses.dataclass
class Case:
    spec: Spec
    seed: int
    num_blocks: int
    poison_block: int
    scale: np.float32
    context_lens: np.ndarray      # int32 [S]; includes the new token
    block_tables: np.ndarray      # int32 [S, MB]; padding -> poison block
    q: np.ndarray                 # [S, Hq, D] act storage dtype
    pre_key: np.ndarray           # [T, Hkv, D] tokens already in context (unique slots)
    pre_value: np.ndarray
    pre_slots: np.ndarray         # int64 [T]
    key: np.ndarray               # [S, Hkv, D] new token of each sequence
    value: np.ndarray
    slot_mapping: np.ndarray      # int64 [S]
    k_scale: Optional[np.ndarray]  # float32 [NB, Hkv] (int8 cache only)
    v_scale: Optional[np.ndarray]
    refcount: np.ndarray          # int32 [NB]

    # convenience ---------------------------------------------------------
    @property
    def S(self):
        return self.spec.num_seqs

    @property
    def Hq(self):
        return self.spec.num_heads

    @property
    def Hkv(self):
        return self.spec.num_kv_heads

    @property
    def D(self):
        return self.spec.head_dim

    @property
    def B(self):
        return self.spec.block_size

    @property
    def MB(self):
        return self.block_tables.shape[1]

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.S else 0

    def empty_pool(self):
        """(k_cache, v_cache) [NB, Hkv, B, D] filled with poison."""
        shape = (self.num_blocks, self.Hkv, self.B, self.D)
        c = self.spec.cache
        if c == "f32":
            k = np.full(shape, F32_POISON, dtype=np.uint32).view(np.float32)
        elif c == "bf16":
            k = np.full(shape, BF16_POISON, dtype=np.uint16)
        else:
            k = np.full(shape, I8_POISON, dtype=np.int8)
        return k, k.copy()

    def scales_or_dummy(self):
        if self.k_scale is not None:
            return self.k_scale, self.v_scale
        return None, None


def _draw_lens(spec: Spec, rng: np.random.Generator) -> np.ndarray:
    kind = spec.lens[0]
    S = spec.num_seqs
    if kind == "fixed":
        L = np.asarray(spec.lens[1], dtype=np.int64)
        assert L.shape == (S,)
    elif kind == "const":
        L = np.full(S, spec.lens[1], dtype=np.int64)
    elif kind == "uniform":
        L = rng.integers(spec.lens[1], spec.lens[2] + 1, size=S)
    elif kind == "lognormal":
        med, sigma, lo, hi = spec.lens[1:]
        L = np.clip(np.rint(rng.lognormal(math.log(med), sigma, size=S)), lo, hi).astype(np.int64)
    else:
        raise ValueError(kind)
    return L.astype(np.int32)


def _cast(x32: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits(x32) if dtype == "bf16" else np.ascontiguousarray(x32, dtype=np.float32)


def make_case(spec: Spec, seed: int) -> Case:
    """Build one seeded decode batch.

    Draw order: context lengths, block permutation, Q, K then V of every
    in-context token (group prefixes first), then the cast to the activation
    dtype. ``context_lens[s]`` counts the new token, which sits at logical
    position ``L-1`` and is written by the decode step itself.
    """
    if spec.act not in ACT_DTYPES or spec.cache not in CACHE_DTYPES:
        raise ValueError("unsupported dtype")
    if spec.num_heads % spec.num_kv_heads:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    rng = np.random.default_rng(seed)
    S, Hkv, D, B = spec.num_seqs, spec.num_kv_heads, spec.head_dim, spec.block_size
    L = _draw_lens(spec, rng)
    if S and (L.min() < 1):
        raise ValueError("every sequence holds at least its new token")
    max_len = spec.max_len or (int(L.max()) if S else 1)
    if S and L.max() > max_len:
        raise ValueError("context length above the spec's bound")
    MB = max(1, -(-max_len // B))
    nblk = -(-L.astype(np.int64) // B)

    prefix = spec.prefix_groups > 0
    if prefix:
        if S % spec.prefix_groups or spec.prefix_tokens % B:
            raise ValueError("prefix groups must split the batch and the prefix must be whole blocks")
        gsz = S // spec.prefix_groups
        pblk = spec.prefix_tokens // B
        shared = np.minimum(pblk, (L.astype(np.int64) - 1) // B)
        need = spec.prefix_groups * pblk + int((nblk - shared).sum())
    else:
        gsz = pblk = 0
        shared = np.zeros(S, dtype=np.int64)
        need = int(nblk.sum())

    if spec.pool[0] == "fixed":
        NB = int(spec.pool[1])
        if NB - 1 < need:
            raise ValueError("fixed pool too small")
    else:
        NB = int(math.ceil(spec.pool[1] * need)) + 1
    pool = BlockPool(NB, rng)

    bt = np.full((S, MB), pool.poison, dtype=np.int32)
    group_ids = []
    for s in range(S):
        if prefix and s % gsz == 0:
            group_ids.append([pool.alloc() for _ in range(pblk)])
        row = []
        if prefix:
            for lb in range(int(shared[s])):
                row.append(pool.share(group_ids[s // gsz][lb]))
        for lb in range(int(shared[s]), int(nblk[s])):
            row.append(pool.alloc())
        bt[s, :len(row)] = row

    q32 = rng.standard_normal((S, spec.num_heads, D), dtype=np.float32)
    if spec.q_std != 1.0:
        q32 = q32 * np.float32(spec.q_std)

    # token values ---------------------------------------------------------
    # Every token to be written (pre: already in context; new: the decode
    # step's token) takes its K/V from a "source" draw. Sources are drawn in
    # order -- group prefixes first, then each sequence's own tokens -- K for
    # all sources, then V, in chunks that are cast and scattered directly into
    # the output arrays.
    if prefix:
        G = spec.prefix_groups
        first_fresh = np.minimum(L.astype(np.int64) - 1, spec.prefix_tokens)
        nfresh = L.astype(np.int64) - first_fresh
        n_src = G * spec.prefix_tokens + int(nfresh.sum())
        fresh_off = G * spec.prefix_tokens + np.concatenate([[0], np.cumsum(nfresh)[:-1]])
        pre_slots, pre_src = [], []
        for g in range(G):
            ids = np.asarray(group_ids[g], dtype=np.int64)
            p = np.arange(spec.prefix_tokens, dtype=np.int64)
            pre_slots.append(ids[p // B] * B + p % B)
            pre_src.append(g * spec.prefix_tokens + p)
        new_slots = np.empty(S, dtype=np.int64)
        new_src = np.empty(S, dtype=np.int64)
        for s in range(S):
            g = s // gsz
            p = np.arange(int(shared[s]) * B, int(L[s]), dtype=np.int64)
            slots = bt[s, p // B].astype(np.int64) * B + p % B
            src = np.where(p < first_fresh[s], g * spec.prefix_tokens + p,
                           fresh_off[s] + (p - first_fresh[s]))
            pre_slots.append(slots[:-1])
            pre_src.append(src[:-1])
            new_slots[s] = slots[-1]
            new_src[s] = src[-1]
        pre_slots = np.concatenate(pre_slots) if pre_slots else np.zeros(0, np.int64)
        pre_src = np.concatenate(pre_src) if pre_src else np.zeros(0, np.int64)
    else:
        n_src = int(L.sum())
        off = np.concatenate([[0], np.cumsum(L.astype(np.int64))[:-1]]) if S else np.zeros(0, np.int64)
        seq_of = np.repeat(np.arange(S), L)
        p = np.arange(n_src, dtype=np.int64) - np.repeat(off, L)
        slots = bt[seq_of, p // B].astype(np.int64) * B + p % B
        is_new = p == np.repeat(L.astype(np.int64) - 1, L)
        pre_slots, pre_src = slots[~is_new], np.nonzero(~is_new)[0]
        new_slots, new_src = slots[is_new], np.nonzero(is_new)[0]

    q = _cast(q32, spec.act)
    T_pre = len(pre_src)
    all_src = np.concatenate([pre_src, new_src]).astype(np.int64)
    order = np.argsort(all_src, kind="stable")
    sorted_src = all_src[order]
    st = storage_dtype(spec.act)
    outs = []
    chunk = max(1, (1 << 21) // max(1, Hkv * D))          # ~2M values per draw
    for _ in range(2):                                      # K, then V
        allv = np.empty((T_pre + S, Hkv, D), dtype=st)
        for a0 in range(0, n_src, chunk):
            a1 = min(n_src, a0 + chunk)
            x = _cast(rng.standard_normal((a1 - a0, Hkv, D), dtype=np.float32), spec.act)
            lo, hi = np.searchsorted(sorted_src, [a0, a1])
            allv[order[lo:hi]] = x[sorted_src[lo:hi] - a0]
        outs.append(allv)
    kall, vall = outs

    case = Case(
        spec=spec, seed=seed, num_blocks=NB, poison_block=pool.poison,
        scale=np.float32(1.0 / math.sqrt(D)),
        context_lens=L, block_tables=bt, q=q,
        pre_key=kall[:T_pre], pre_value=vall[:T_pre], pre_slots=pre_slots.astype(np.int64),
        key=kall[T_pre:], value=vall[T_pre:], slot_mapping=new_slots.astype(np.int64),
        k_scale=None, v_scale=None, refcount=pool.refcount.copy(),
    )
    if spec.cache == "i8":
        case.k_scale, case.v_scale = absmax_scales(case)
    check_cow(case)
    return case


@dataclasses.dataclass
class Queries:
    """Several new query tokens per sequence: rows query_start_loc[s] ..
    query_start_loc[s + 1] - 1 of ``q`` are the newest n_s tokens of sequence
    s (positions L_s - n_s .. L_s - 1, already in its context)."""
    query_start_loc: np.ndarray    # int32 [S + 1]
    q: np.ndarray                  # [T, Hq, D], activation storage dtype
    q_lens: np.ndarray             # int64 [S], n_s

    @property
    def num_tokens(self) -> int:
        return int(self.query_start_loc[-1])


def query_counts(context_lens: np.ndarray, q_lens, rng: np.random.Generator) -> np.ndarray:
    """Per-sequence query-row counts n_s (int64 [S]) for ``make_queries``:
    ("const", n), ("uniform", lo, hi) (inclusive, drawn from ``rng``) or a
    sequence of counts, each clipped to [0, L_s]."""
    L = np.asarray(context_lens).astype(np.int64)
    S = L.shape[0]
    if isinstance(q_lens, tuple) and q_lens[0] == "const":
        n = np.full(S, int(q_lens[1]), dtype=np.int64)
    elif isinstance(q_lens, tuple) and q_lens[0] == "uniform":
        n = rng.integers(q_lens[1], q_lens[2] + 1, size=S).astype(np.int64)
    else:
        n = np.asarray(q_lens, dtype=np.int64).reshape(S)
    return np.clip(n, 0, L)


def draw_lens(spec: Spec, seed: int) -> np.ndarray:
    """The context lengths ``make_case(spec, seed)`` draws (its first draw),
    without building the batch."""
    return _draw_lens(spec, np.random.default_rng(seed))


def make_queries(case: Case, q_lens, seed: int) -> Queries:
    """Queries for a multi-token step over ``case``'s cache.

    ``q_lens``: ("const", n), ("uniform", lo, hi) (inclusive) or a sequence
    of per-sequence counts; each count is clipped to [0, L_s]. Q ~ N(0, 1)
    times the spec's q_std, cast to the activation dtype."""
    rng = np.random.default_rng(seed)
    S = case.S
    n = query_counts(case.context_lens, q_lens, rng)
    qsl = np.zeros(S + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(n)
    q32 = rng.standard_normal((int(qsl[-1]), case.Hq, case.D), dtype=np.float32)
    if case.spec.q_std != 1.0:
        q32 = q32 * np.float32(case.spec.q_std)
    return Queries(query_start_loc=qsl, q=_cast(q32, case.spec.act), q_lens=n)


# Multi-token workloads over paged caches: the speculative verify of K + 1 = 4
# tokens per sequence on the Llama-shaped batch and on the long-context batch
# (split over 512-token partitions), and 512-token prefill chunks appended to 8
# cached 3584-token prefixes (contexts of 4096).
MULTI_QUERY = {
    "verify": (CONFIGS[2], ("const", 4)),
    "verify_long": (CONFIGS[3], ("const", 4)),
    "prefill": (Spec("chunked prefill bf16", 8, ("const", 4096), 32, 8, 128, 16,
                     act="bf16", cache="bf16", max_len=4096), ("const", 512)),
}


def absmax_scales(case: Case):
    """Caller-side int8 scales: absmax/127 over everything written into each
    (block, kv head), in fp32; 1.0 where absmax is 0 or the block is unused."""
    NB, Hkv, B = case.num_blocks, case.Hkv, case.B
    out = []
    rows = max(1, (1 << 21) // max(1, Hkv * case.D))
    for pre, new in ((case.pre_key, case.key), (case.pre_value, case.value)):
        amax = np.zeros((NB, Hkv), dtype=np.float32)
        for vals, slots in ((pre, case.pre_slots), (new, case.slot_mapping)):
            for r0 in range(0, len(slots), rows):
                a = np.abs(as_f32(vals[r0:r0 + rows], case.spec.act)).max(axis=2)   # [T, Hkv]
                np.maximum.at(amax, slots[r0:r0 + rows] // B, a)
        sc = amax / np.float32(127.0)
        sc[amax == 0] = np.float32(1.0)
        out.append(sc.astype(np.float32))
    return out[0], out[1]


def check_cow(case: Case) -> None:
    """The decode-step write never lands in a shared block."""
    if len(case.slot_mapping) == 0:
        return
    blocks = case.slot_mapping[case.slot_mapping >= 0] // case.B
    if (case.refcount[blocks] != 1).any():
        raise AssertionError("slot_mapping targets a shared block")


# --------------------------------------------------------------------------
# Placement transforms (for invariance tests)
# --------------------------------------------------------------------------

def permute_placement(case: Case, seed: int) -> Case:
    """Same logical content, physical blocks renamed by a random permutation."""
    rng = np.random.default_rng(seed)
    NB = case.num_blocks
    perm = np.arange(NB)
    perm[:NB - 1] = rng.permutation(NB - 1)    # poison block keeps its id
    B = case.B

    def remap(slots):
        return (perm[slots // B] * B + slots % B).astype(np.int64)

    inv = np.empty(NB, dtype=np.int64)
    inv[perm] = np.arange(NB)
    new = dataclasses.replace(
        case,
        block_tables=perm[case.block_tables].astype(np.int32),
        pre_slots=remap(case.pre_slots),
        slot_mapping=remap(case.slot_mapping),
        refcount=case.refcount[inv],
    )
    if case.k_scale is not None:
        new.k_scale = case.k_scale[inv]
        new.v_scale = case.v_scale[inv]
    return new


def unshare_prefixes(case: Case) -> Case:
    """Give every sequence private copies of the blocks it shares (a pool with
    no copy-on-write), leaving every logical token's values unchanged."""
    S, B = case.S, case.B
    nblk = -(-case.context_lens.astype(np.int64) // B)
    NB0 = case.num_blocks
    # which (seq, logical block) entries point at a block used by more than one table row
    uses = np.zeros(NB0, dtype=np.int64)
    for s in range(S):
        np.add.at(uses, case.block_tables[s, :nblk[s]].astype(np.int64), 1)
    extra = [(s, lb) for s in range(S) for lb in range(int(nblk[s]))
             if uses[case.block_tables[s, lb]] > 1]
    NB = NB0 + len(extra)
    poison = NB - 1
    bt = case.block_tables.astype(np.int64).copy()
    bt[bt == case.poison_block] = poison
    copy_of = {}
    nxt = NB0 - 1                    # old poison id becomes an ordinary block id
    for (s, lb) in extra:
        copy_of[(s, lb)] = (int(bt[s, lb]), nxt)
        bt[s, lb] = nxt
        nxt += 1
    assert nxt == NB - 1
    # every token written into a shared block is re-written into each private copy
    pre_blocks = case.pre_slots // B
    add_slots, add_src = [], []
    for (s, lb), (old, newb) in copy_of.items():
        m = np.nonzero(pre_blocks == old)[0]
        add_slots.append(newb * B + case.pre_slots[m] % B)
        add_src.append(m)
    keep = ~np.isin(pre_blocks, list({o for (o, _) in copy_of.values()}))
    pre_slots = np.concatenate([case.pre_slots[keep]] + add_slots)
    src = np.concatenate([np.nonzero(keep)[0]] + add_src)
    refcount = np.zeros(NB, dtype=np.int32)
    for s in range(S):
        refcount[bt[s, :nblk[s]]] = 1
    new = dataclasses.replace(
        case, num_blocks=NB, poison_block=poison,
        block_tables=bt.astype(np.int32), pre_slots=pre_slots.astype(np.int64),
        pre_key=case.pre_key[src], pre_value=case.pre_value[src], refcount=refcount,
    )
    if case.k_scale is not None:
        ks = np.ones((NB, case.Hkv), np.float32)
        vs = np.ones((NB, case.Hkv), np.float32)
        ks[:NB0 - 1] = case.k_scale[:NB0 - 1]
        vs[:NB0 - 1] = case.v_scale[:NB0 - 1]
        for (s, lb), (old, newb) in copy_of.items():
            ks[newb] = case.k_scale[old]
            vs[newb] = case.v_scale[old]
        new.k_scale, new.v_scale = ks, vs
    return new


# --------------------------------------------------------------------------
# Byte accounting
# --------------------------------------------------------------------------

def in_context_slots(case: Case) -> np.ndarray:
    """Physical slot of every (sequence, logical token) in context."""
    B = case.B
    L = case.context_lens.astype(np.int64)
    seq_of = np.repeat(np.arange(case.S), L)
    off = np.concatenate([[0], np.cumsum(L)[:-1]]) if case.S else np.zeros(0, np.int64)
    p = np.arange(int(L.sum()), dtype=np.int64) - np.repeat(off, L)
    return case.block_tables[seq_of, p // B].astype(np.int64) * B + p % B


def traffic(case: Case) -> dict:
    """Algorithmic bytes of one decode step (what the method must move).

    KV counts each unique physical in-context token once (shared prefixes are
    read from HBM once at best); ``kv_logical`` counts every (seq, token).
    """
    sp = case.spec
    ce, ae = elt_bytes(sp.cache), elt_bytes(sp.act)
    Hkv, D, S, Hq = case.Hkv, case.D, case.S, case.Hq
    slots = in_context_slots(case)
    uniq = int(np.unique(slots).size)
    logical = int(slots.size)
    per_tok = 2 * Hkv * D * ce
    nblk = -(-case.context_lens.astype(np.int64) // case.B)
    scales = 0
    if sp.cache == "i8":
        used = np.unique(np.concatenate([case.block_tables[s, :nblk[s]] for s in range(S)]))
        scales = int(used.size) * Hkv * 2 * 4
    decode = {
        "kv": uniq * per_tok,
        "kv_logical": logical * per_tok,
        "q": S * Hq * D * ae,
        "out": S * Hq * D * ae,
        "block_tables": int(nblk.sum()) * 4,
        "context_lens": 4 * S,
        "scales": scales,
    }
    decode["total"] = sum(v for k, v in decode.items() if k != "kv_logical")
    write = 2 * len(case.slot_mapping) * Hkv * D * (ae + ce) + 8 * len(case.slot_mapping)
    return {"decode": decode, "write": write, "unique_tokens": uniq, "logical_tokens": logical,
            "sum_len": int(case.context_lens.sum()),
            "flops": 4 * D * Hq * int(case.context_lens.sum())}
