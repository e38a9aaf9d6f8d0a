"""RoPE positions that are not the token's index in its request, on the GPU against the oracle.

The ABI takes each token's RoPE position as its own input (`positions`), apart
from the cache slot the token is written to (its index in the request, or
P_r + j, or L_b).  Every other parity test uses positions equal to those slots,
so these cases pin that the kernels rotate by `positions` and place by slot.
"""

import numpy as np
import pytest
import torch

from harness import check_prefill_caches, f64, assert_close, note, oracle_prefill, run_prefill, tol_for
from test_parity_append import _check_append
from test_parity_decode import _check_decode
from workloads import HeadConfig, make_append_inputs, make_decode_inputs, make_prefill_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _random_positions(n: int, seed: int) -> torch.Tensor:
    # Unsorted, repeated and far from the slots: 0 .. 40000.
    g = torch.Generator().manual_seed(seed)
    return torch.randint(0, 40000, (n,), generator=g, dtype=torch.int32).to(DEV)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
@pytest.mark.parametrize("hq,hkv,d", [(16, 4, 128), (8, 2, 64)], ids=["d128", "d64"])
def test_prefill_rotates_by_positions(hq, hkv, d, dtype):
    h = HeadConfig(hq, hkv, d, 1e-6, 1e6)
    lens = [37, 0, 70, 1, 129]
    p = make_prefill_inputs(h, lens, seed=31, dtype=dtype, device=DEV, capacity=max(lens))
    p.positions = _random_positions(p.num_tokens, 32)
    note(f"prefill hq{hq} hkv{hkv} d{d} {dtype}, positions {p.positions[:5].tolist()}...")
    k0, v0 = p.k_cache.clone(), p.v_cache.clone()
    got = run_prefill(p)
    ref = oracle_prefill(p)
    tol = tol_for(dtype)
    assert_close(f64(got["out"]), ref["out"], tol, "out")
    check_prefill_caches(p, k0, v0, ref, tol)
    # The slot order is unchanged: a different positions array changes the output.
    p2 = make_prefill_inputs(h, lens, seed=31, dtype=dtype, device=DEV, capacity=max(lens))
    assert not np.allclose(f64(run_prefill(p2)["out"]), f64(got["out"]), atol=tol)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_decode_rotates_by_positions(dtype):
    h = HeadConfig(32, 8, 128, 1e-6, 1e6)
    d = make_decode_inputs(h, [0, 5, 300, 1023, 17], seed=33, dtype=dtype, device=DEV)
    d.positions = _random_positions(d.num_seqs, 34)
    note(f"decode {dtype}, positions {d.positions.tolist()} for cache lengths {d.cache_lens.tolist()}")
    _check_decode(d)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_append_rotates_by_positions(dtype):
    h = HeadConfig(16, 4, 128, 1e-6, 1e6)
    a = make_append_inputs(h, [0, 40, 100], [30, 65, 1], seed=35, dtype=dtype, device=DEV)
    a.positions = _random_positions(a.num_tokens, 36)
    note(f"append {dtype}, positions {a.positions[:5].tolist()}...")
    _check_append(a)
