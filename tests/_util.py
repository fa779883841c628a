"""Test helpers: tensor <-> bit-pattern conversion and one oracle run per
workload.  No arithmetic of the epilogue lives here."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from mla_decode_concat_amd import inputs as I


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw bit patterns of a CPU tensor: bf16/fp16 -> uint16, e4m3 -> uint8."""
    t = t.detach().cpu().contiguous()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype in (torch.float8_e4m3fn, torch.uint8):
        return t.view(torch.uint8).numpy()
    raise TypeError(t.dtype)


def oracle_run(w: I.Workload, inp: dict, cache_init: np.ndarray | None = None):
    """Run the oracle on the workload's inputs; returns (q_out, cache) as bit
    arrays [T,H,576] and [NB,BS,576]."""
    T, H = w.tokens, w.heads
    q = np.zeros((T, H, I.ROW), dtype=np.uint8 if w.q_fp8 else np.uint16)
    cache = bits(inp["cache"]).copy() if cache_init is None else cache_init.copy()
    pos = inp["positions"].numpy() if inp["positions"] is not None else None
    cs = inp["rope_cos_sin"]
    if cs is not None:
        cs = bits(cs) if cs.dtype == torch.bfloat16 else cs.numpy()
    oracle.insert(q, bits(inp["ql_nope"]), bits(inp["q_pe"]), bits(inp["kv_c"]),
                  bits(inp["k_pe"]), cache, inp["slot_mapping"].numpy(), pos, cs,
                  w.q_scale, w.kv_scale, w.rope, w.q_fp8, w.kv_fp8,
                  fp16=w.dtype == "fp16", gptj=w.rope_style == "gptj")
    return q, cache
