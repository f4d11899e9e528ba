"""Exactness probes shared by the GPU parity tests (harness side only: they
build inputs and expected values from the source draws; no attention
arithmetic)."""
from __future__ import annotations

import dataclasses

import numpy as np

import pins
import synth


def onehot_case(spec, seed, pick, max_pos=None):
    """A batch whose output is one V row exactly: q = 128 e_0 for every query
    head, k_{t*}[:, 0] = 128 and k_t[:, 0] = 0 for every other token t, so the
    logit of t* exceeds every other by 16384 * scale (> 745 in natural units for
    head_dim <= 256) and every other softmax weight underflows to exactly 0.

    ``pick(s, candidates)`` chooses t* for sequence s among the tokens in blocks
    that s owns alone (a probe in a shared copy-on-write block would be seen by
    the whole group), limited to positions <= max_pos(s) when given. int8
    caches get absmax scales over the probed values. Returns (case, t*s)."""
    case = synth.make_case(spec, seed)
    act = spec.act
    idx, _, _ = pins.source_rows(case)
    npre = len(case.pre_slots)
    one = np.float32(128.0)
    val = synth.bf16_bits(np.array([one]))[0] if act == "bf16" else one
    zero = np.uint16(0) if act == "bf16" else np.float32(0)
    pk, nk, q = case.pre_key.copy(), case.key.copy(), np.zeros_like(case.q)
    pk[:, :, 0] = zero
    nk[:, :, 0] = zero
    q[:, :, 0] = val
    ts = []
    for s in range(case.S):
        L = int(case.context_lens[s])
        hi = L - 1 if max_pos is None else min(L - 1, int(max_pos(s)))
        own = [t for t in range(hi + 1)
               if case.refcount[case.block_tables[s, t // case.B]] == 1]
        t = own[pick(s, len(own))]
        ts.append(t)
        slot = int(case.block_tables[s, t // case.B]) * case.B + t % case.B
        r = idx[slot]
        if r < npre:
            pk[r, :, 0] = val
        else:
            nk[r - npre, :, 0] = val
    new = dataclasses.replace(case, pre_key=pk, key=nk, q=q)
    if spec.cache == "i8":
        new.k_scale, new.v_scale = synth.absmax_scales(new)
    return new, ts


def onehot_queries(case, q_lens):
    """Query rows for a several-rows-per-sequence step over ``case``: q = 128 e_0
    on every row and head (the one-hot probe's query), row counts q_lens."""
    n = np.asarray(q_lens, dtype=np.int64)
    qsl = np.zeros(case.S + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(n)
    q = np.zeros((int(qsl[-1]), case.Hq, case.D), dtype=case.q.dtype)
    q[:, :, 0] = case.q[0, 0, 0]                     # the probe's 128
    return synth.Queries(query_start_loc=qsl, q=q, q_lens=n)
