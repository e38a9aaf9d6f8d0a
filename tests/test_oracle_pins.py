"""The oracle against closed forms, stated invariants, independent evaluators and printed shapes."""

import pytest

import oracle.layer_ops as lo
import oracle.qknorm_rope_attn as orc
import pins


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_pin(check):
    check(orc)


@pytest.mark.parametrize("check", pins.LAYER_OPS_CHECKS, ids=lambda c: c.__name__)
def test_layer_ops_pin(check):
    check(lo)


def test_round_to_bf16_matches_torch():
    import numpy as np
    import torch

    r = np.random.default_rng(0)
    x = np.concatenate([r.standard_normal(10000) * 10, [0.0, -0.0, 1.0, 3.0e38, 1e-40, 1.00390625, 1.01171875]])
    want = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(orc.round_to_bf16(x), want)


@pytest.mark.parametrize("check", pins.PAGED_CHECKS, ids=lambda c: c.__name__)
def test_paged_pin(check):
    import oracle.paged as pg

    check(pg)
