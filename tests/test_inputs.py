"""The seeded input recipes (no GPU): shapes, dtypes, slot and position
ranges, and reproducibility, for the host generator and for the device
generator used by the maximum-size test (run here on the CPU device)."""
from __future__ import annotations

import pytest
import torch

from mla_decode_concat_amd import inputs as I


def _check_recipe(w: I.Workload, d: dict):
    T, H = w.tokens, w.heads
    act = w.torch_dtype
    assert d["ql_nope"].shape == (T, H, 512) and d["ql_nope"].dtype == act
    assert d["q_pe"].shape == (T, H, 64) and d["q_pe"].dtype == act
    assert d["kv_c"].shape == (T, 512) and d["kv_c"].dtype == act
    assert d["k_pe"].shape == (T, 64) and d["k_pe"].dtype == act
    slots = d["slot_mapping"].cpu()
    assert slots.dtype == torch.int64 and slots.shape == (T,)
    assert int(slots.min()) >= 0 and int(slots.max()) < w.num_slots
    assert torch.unique(slots).numel() == T                 # a prefix of a permutation
    cache = d["cache"]
    assert cache.shape == (w.num_blocks, w.block_size, 576)
    assert int(cache.view(torch.uint8).count_nonzero()) == 0
    if w.rope:
        pos = d["positions"].cpu()
        assert pos.dtype == torch.int64 and pos.shape == (T,)
        assert int(pos.min()) >= 0 and int(pos.max()) < w.max_position
        assert d["rope_cos_sin"].shape == (w.max_position, 64)
    else:
        assert d["positions"] is None and d["rope_cos_sin"] is None
    x = d["ql_nope"].float()
    assert abs(float(x.mean())) < 0.05 and abs(float(x.std()) - 1.0) < 0.05   # N(0, 1)


@pytest.mark.parametrize("rope", [False, True])
def test_host_recipe(rope):
    w = I.custom(200, 16, rope=rope, q_fp8=True, kv_fp8=True)
    a, b = I.make_inputs(w, seed=5), I.make_inputs(w, seed=5)
    _check_recipe(w, a)
    assert all(torch.equal(a[k], b[k]) for k in ("ql_nope", "q_pe", "kv_c", "k_pe", "slot_mapping"))


@pytest.mark.parametrize("rope", [False, True])
def test_device_recipe_on_the_cpu_device(rope):
    w = I.custom(200, 16, rope=rope, q_fp8=True, kv_fp8=True)
    a = I.make_inputs_on_device(w, "cpu", seed=5, chunk=1000)
    b = I.make_inputs_on_device(w, "cpu", seed=5, chunk=1000)
    _check_recipe(w, a)
    assert all(torch.equal(a[k], b[k]) for k in ("ql_nope", "q_pe", "kv_c", "k_pe", "slot_mapping"))
    c = I.make_inputs_on_device(w, "cpu", seed=6, chunk=1000)
    assert not torch.equal(a["ql_nope"], c["ql_nope"])


def _check_uk_recipe(w: I.Workload, d: dict):
    T, H = w.tokens, w.heads
    assert d["q_b"].shape == (T, H, 192) and d["q_b"].dtype == w.torch_dtype
    assert d["q_nope"].data_ptr() == d["q_b"].data_ptr() and d["q_nope"].shape == (T, H, 128)
    assert d["q_pe"].data_ptr() == d["q_b"].data_ptr() + 128 * d["q_b"].element_size()
    assert d["q_nope"].stride() == (H * 192, 192, 1) and d["q_pe"].stride() == (H * 192, 192, 1)
    assert d["w_uk_t"].shape == (H, 512, 128) and d["w_uk_t"].dtype == w.torch_dtype
    wt = d["w_uk_t"].float()
    assert abs(float(wt.std()) * 128 ** 0.5 - 1.0) < 0.05      # N(0, 1/128)
    x = d["q_b"].float()
    assert abs(float(x.mean())) < 0.05 and abs(float(x.std()) - 1.0) < 0.05
    assert "ql_nope" not in d
    rest = dict(d, ql_nope=torch.zeros(T, H, 512, dtype=w.torch_dtype))
    rest["ql_nope"].normal_()
    _check_recipe(w, rest)


@pytest.mark.parametrize("rope", [False, True])
def test_uk_recipes_host_and_device(rope):
    w = I.custom(200, 16, rope=rope, q_fp8=True, kv_fp8=True)
    h = I.make_uk_inputs(w, seed=5)
    _check_uk_recipe(w, {k: v for k, v in h.items() if k != "ql_nope"})
    a = I.make_inputs_on_device(w, "cpu", seed=5, chunk=1000, uk=True)
    b = I.make_inputs_on_device(w, "cpu", seed=5, chunk=1000, uk=True)
    _check_uk_recipe(w, a)
    assert all(torch.equal(a[k], b[k]) for k in ("q_b", "w_uk_t", "kv_c", "k_pe", "slot_mapping"))
