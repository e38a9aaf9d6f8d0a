"""A seeded sweep of small random configurations, on the GPU against the oracle.

Each case draws head counts (every GQA width the kernels tile: G = 1..16),
the head dimension, eps, the RoPE base, ragged and empty lengths and, for
some, RoPE positions apart from the cache slots.  Deterministic (fixed seeds),
sized so the oracle finishes each case in well under a second.
"""

import random

import pytest
import torch

from harness import assert_close, check_prefill_caches, f64, note, oracle_prefill, run_prefill, tol_for
from test_parity_append import _check_append
from test_parity_decode import _check_decode
from workloads import HeadConfig, make_append_inputs, make_decode_inputs, make_prefill_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
CASES = 12
GROUPS = [1, 2, 3, 4, 5, 6, 8, 12, 16]


def _heads(rng: random.Random) -> HeadConfig:
    g = rng.choice(GROUPS)
    hkv = rng.choice([h for h in (1, 2, 4, 8) if g * h <= 64])
    return HeadConfig(g * hkv, hkv, rng.choice([64, 128]), rng.choice([1e-6, 1e-5, 1e-3]),
                      rng.choice([1e4, 5e5, 1e6]))


def _maybe_positions(rng: random.Random, n: int):
    if rng.random() < 0.5:
        return None
    g = torch.Generator().manual_seed(rng.randrange(1 << 30))
    return torch.randint(0, 50000, (n,), generator=g, dtype=torch.int32).to(DEV)


def _label(kind, i, h, extra):
    return f"{kind} case {i}: Hq {h.num_q_heads} Hkv {h.num_kv_heads} D {h.head_dim} eps {h.rms_eps} " \
           f"base {h.rope_base} {extra}"


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
@pytest.mark.parametrize("i", range(CASES))
def test_prefill_sweep(i, dtype):
    rng = random.Random(1000 + i)
    h = _heads(rng)
    lens = [rng.choice([0, 1, rng.randint(2, 64), rng.randint(65, 300)]) for _ in range(rng.randint(1, 6))]
    if sum(lens) == 0:
        lens[0] = 1
    p = make_prefill_inputs(h, lens, seed=rng.randrange(1 << 20), dtype=dtype, device=DEV,
                            capacity=max(lens) + rng.randint(0, 9))
    pos = _maybe_positions(rng, p.num_tokens)
    if pos is not None:
        p.positions = pos
    note(_label("prefill", i, h, f"lens {lens} positions {'random' if pos is not None else 'slots'}"))
    k0, v0 = p.k_cache.clone(), p.v_cache.clone()
    got = run_prefill(p)
    ref = oracle_prefill(p)
    tol = tol_for(dtype)
    assert_close(f64(got["out"]), ref["out"], tol, "out")
    check_prefill_caches(p, k0, v0, ref, tol)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
@pytest.mark.parametrize("i", range(CASES))
def test_append_sweep(i, dtype):
    rng = random.Random(2000 + i)
    h = _heads(rng)
    b = rng.randint(1, 5)
    past = [rng.choice([0, rng.randint(1, 64), rng.randint(65, 500)]) for _ in range(b)]
    chunks = [rng.choice([0, 1, rng.randint(2, 64), rng.randint(65, 200)]) for _ in range(b)]
    if sum(chunks) == 0:
        chunks[0] = 1
    a = make_append_inputs(h, past, chunks, seed=rng.randrange(1 << 20), dtype=dtype, device=DEV)
    pos = _maybe_positions(rng, a.num_tokens)
    if pos is not None:
        a.positions = pos
    note(_label("append", i, h, f"past {past} chunks {chunks}"))
    _check_append(a)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
@pytest.mark.parametrize("i", range(CASES))
def test_decode_sweep(i, dtype):
    rng = random.Random(3000 + i)
    h = _heads(rng)
    lens = [rng.choice([0, 1, rng.randint(2, 100), rng.randint(101, 2000)]) for _ in range(rng.randint(1, 8))]
    d = make_decode_inputs(h, lens, seed=rng.randrange(1 << 20), dtype=dtype, device=DEV)
    pos = _maybe_positions(rng, d.num_seqs)
    if pos is not None:
        d.positions = pos
    note(_label("decode", i, h, f"cache lengths {lens}"))
    _check_decode(d)


@pytest.mark.parametrize("i", range(CASES))
def test_prefill_sweep_running_max_kernel(i):
    """The same kind of random cases in bf16, with one element of each norm weight raised to 2.5 so that
    max|w_q| max|w_k| exceeds the bound under which the unshifted kernel runs: a plain prefill then goes through
    the running-max kernel, for every query-head grouping it is instantiated for.  The outlier moves only the
    bound, not the typical score."""
    import numpy as np
    rng = random.Random(3000 + i)
    h = _heads(rng)
    lens = [rng.choice([0, 1, rng.randint(2, 64), rng.randint(65, 300)]) for _ in range(rng.randint(1, 6))]
    if sum(lens) == 0:
        lens[0] = 1
    p = make_prefill_inputs(h, lens, seed=rng.randrange(1 << 20), dtype=torch.bfloat16, device=DEV,
                            capacity=max(lens) + rng.randint(0, 9))
    d = h.head_dim
    for w, at, sign in ((p.q_norm_weight, rng.randrange(d), 1.0), (p.k_norm_weight, rng.randrange(d), -1.0)):
        w[at] = sign * 2.5
    assert float(p.q_norm_weight.abs().max()) * float(p.k_norm_weight.abs().max()) > 4.1
    note(_label("prefill (running max)", i, h, f"lens {lens}"))
    k0, v0 = p.k_cache.clone(), p.v_cache.clone()
    got = run_prefill(p)
    ref = oracle_prefill(p)
    assert_close(f64(got["out"]), ref["out"], tol_for(torch.bfloat16), "out")
    # K cache: the bound plus half a bf16 step of the value (the outlier element of k~ can pass 8).
    cu = p.cu_seqlens.cpu().tolist()
    for r in range(p.num_seqs):
        lo, hi = cu[r], cu[r + 1]
        got_k = f64(p.k_cache[r, :, : hi - lo])
        want = np.transpose(ref["k_tilde"][lo:hi], (1, 0, 2))
        assert np.all(np.abs(got_k - want) <= 2e-2 + np.abs(want) * 2.0**-8), f"K cache request {r}"
