"""Move a ``synth.Case`` onto the GPU and run the HIP path on it through the
C ABI (via the thin Python binding). Test/bench plumbing only: it holds no
attention arithmetic."""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

import paged_kv_decode_03_amd as pa
import synth

TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "i8": torch.int8}
TOL = {"f32": 1e-5, "bf16": 2e-2, "i8": 3e-2}


def tol(case) -> float:
    return TOL["i8"] if case.spec.cache == "i8" else TOL[case.spec.act]


def host_to_dev(a: np.ndarray, dtype: str, device) -> torch.Tensor:
    """numpy storage array (float32 / uint16 bf16 bits / int8) -> device tensor."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(
            torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def dev_to_host(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> numpy storage array with the same bits."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def as_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


@dataclasses.dataclass
class DevCase:
    case: synth.Case
    q: torch.Tensor
    block_tables: torch.Tensor
    context_lens: torch.Tensor
    pre_key: torch.Tensor
    pre_value: torch.Tensor
    pre_slots: torch.Tensor
    key: torch.Tensor
    value: torch.Tensor
    slot_mapping: torch.Tensor
    k_scale: torch.Tensor | None
    v_scale: torch.Tensor | None
    k_cache: torch.Tensor | None = None
    v_cache: torch.Tensor | None = None


def to_device(case: synth.Case, device="cuda") -> DevCase:
    act = case.spec.act
    return DevCase(
        case=case,
        q=host_to_dev(case.q, act, device),
        block_tables=torch.from_numpy(case.block_tables).to(device),
        context_lens=torch.from_numpy(case.context_lens).to(device),
        pre_key=host_to_dev(case.pre_key, act, device),
        pre_value=host_to_dev(case.pre_value, act, device),
        pre_slots=torch.from_numpy(case.pre_slots).to(device),
        key=host_to_dev(case.key, act, device),
        value=host_to_dev(case.value, act, device),
        slot_mapping=torch.from_numpy(case.slot_mapping).to(device),
        k_scale=None if case.k_scale is None else torch.from_numpy(case.k_scale).to(device),
        v_scale=None if case.v_scale is None else torch.from_numpy(case.v_scale).to(device),
    )


def poison_pool(case: synth.Case, device="cuda"):
    shape = (case.num_blocks, case.Hkv, case.B, case.D)
    dt = TORCH_DT[case.spec.cache]
    fill = -128 if case.spec.cache == "i8" else float("nan")
    return torch.full(shape, fill, dtype=dt, device=device), torch.full(shape, fill, dtype=dt,
                                                                        device=device)


def fill_pool(dc: DevCase, device="cuda"):
    """Pool as the HIP write leaves it: poison, every in-context token, then
    the new token of each sequence (two pa_write_kv_cache calls)."""
    k, v = poison_pool(dc.case, device)
    if dc.pre_slots.numel():
        pa.write_kv_cache(dc.pre_key, dc.pre_value, k, v, dc.pre_slots, dc.k_scale, dc.v_scale)
    write_new(dc, k, v)
    dc.k_cache, dc.v_cache = k, v
    return k, v


def write_new(dc: DevCase, k, v):
    pa.write_kv_cache(dc.key, dc.value, k, v, dc.slot_mapping, dc.k_scale, dc.v_scale)


def run_decode(dc: DevCase, partition_size=0, k=None, v=None, ws=None, max_context_len=None,
               balanced=False):
    k = dc.k_cache if k is None else k
    v = dc.v_cache if v is None else v
    c = dc.case
    maxL = c.max_context_len if max_context_len is None else max_context_len
    return pa.paged_attention(dc.q, k, v, dc.block_tables, dc.context_lens, float(c.scale), maxL,
                              partition_size, dc.k_scale, dc.v_scale, ws=ws, balanced=balanced)
