"""The configuration's rms_eps and RoPE base reach every kernel, on the GPU against the oracle.

The other parity cases use eps 1e-6 and bases 1e4 / 1e6; here eps is 0.05 (it
moves each row's norm by a few percent) and the base 5e5, so a kernel that
ignored either would fail.
"""

import numpy as np
import pytest
import torch

from harness import assert_close, check_prefill_caches, f64, note, oracle_prefill, run_prefill, tol_for
from test_parity_append import _check_append
from test_parity_decode import _check_decode
from workloads import HeadConfig, make_append_inputs, make_decode_inputs, make_prefill_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
EPS, BASE = 0.05, 5e5


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_prefill_uses_eps_and_base(dtype):
    h = HeadConfig(16, 4, 128, EPS, BASE)
    lens = [90, 3, 200]
    p = make_prefill_inputs(h, lens, seed=41, dtype=dtype, device=DEV, capacity=max(lens))
    note(f"prefill eps {EPS} base {BASE} {dtype}")
    k0, v0 = p.k_cache.clone(), p.v_cache.clone()
    got = run_prefill(p)
    ref = oracle_prefill(p)
    tol = tol_for(dtype)
    assert_close(f64(got["out"]), ref["out"], tol, "out")
    check_prefill_caches(p, k0, v0, ref, tol)
    # The same inputs under eps 1e-6 give a different cache: eps is not a constant.
    q = make_prefill_inputs(HeadConfig(16, 4, 128, 1e-6, BASE), lens, seed=41, dtype=dtype, device=DEV,
                            capacity=max(lens))
    run_prefill(q)
    assert not np.allclose(f64(q.k_cache), f64(p.k_cache), atol=tol)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_decode_uses_eps_and_base(dtype):
    d = make_decode_inputs(HeadConfig(32, 8, 128, EPS, BASE), [0, 77, 3000], seed=43, dtype=dtype, device=DEV)
    note(f"decode eps {EPS} base {BASE} {dtype}")
    _check_decode(d)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_append_uses_eps_and_base(dtype):
    a = make_append_inputs(HeadConfig(8, 2, 64, EPS, BASE), [50, 0], [70, 33], seed=45, dtype=dtype, device=DEV)
    note(f"append eps {EPS} base {BASE} {dtype}")
    _check_append(a)
