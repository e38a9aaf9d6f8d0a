"""Decode on the GPU, through the C ABI, against the fp64 oracle."""

import numpy as np
import pytest
import torch

import oracle
from harness import (BF16_TOL, assert_close, bits, check_decode_result, f64, layer_kw, note, oracle_prefill,
                     run_decode, run_prefill, tol_for)
from workloads import HeadConfig, build_workload, make_decode_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _check_decode(d, subset=None, tol=None):
    """Runs the HIP decode on all requests and checks `subset` of them against the oracle (all if None); every
    new V slot is checked bit for bit and every other slot must keep its bits."""
    tol = tol if tol is not None else tol_for(d.qkv.dtype)
    k_before, v_before = d.k_cache.clone(), d.v_cache.clone()
    got = run_decode(d)
    return check_decode_result(d, got["out"], k_before, v_before, tol, requests=subset)


# (Hq, Hkv, D, cache lengths): split edges (512 keys per split), 16-key step
# edges, empty caches (the token attends to itself only), every GQA width.
CASES = [
    (4, 2, 64, [0, 1, 5, 64]),
    (32, 8, 128, [0, 1, 15, 16, 17, 511, 512, 513, 1000, 2047]),
    (16, 8, 128, [100, 3000]),
    (8, 8, 64, [700, 1]),
    (16, 2, 128, [33, 1025]),
    (12, 4, 64, [50, 600]),
    # query heads per matrix tile (bf16): 16, 12, 10 (two tiles per KV head), 5
    (48, 3, 128, [300, 5]),
    (12, 1, 64, [31, 32, 33]),
    (20, 1, 128, [250, 0]),
    (10, 2, 64, [90, 1100]),
]


def _ids(case):
    hq, hkv, d, lens = case
    return f"hq{hq}-hkv{hkv}-d{d}-L{'_'.join(map(str, lens))}"


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_decode_matches_oracle(case, dtype):
    hq, hkv, d, lens = case
    h = HeadConfig(hq, hkv, d, 1e-6, 1e6)
    note(f"decode {_ids(case)} {dtype}")
    dec = make_decode_inputs(h, lens, seed=sum(lens) % 9973, dtype=dtype, device=DEV, capacity=max(lens) + 4)
    _check_decode(dec)


def test_decode_cache_filled_to_capacity():
    # The new token goes to the last slot of the cache (L_b = capacity - 1).
    h = HeadConfig(32, 8, 128, 1e-6, 1e6)
    dec = make_decode_inputs(h, [95, 40, 0], seed=21, device=DEV, capacity=96)
    _check_decode(dec)


def test_decode_many_short_requests():
    # 600 requests x 8 KV heads of 1-7 steps: each wavefront's range of steps
    # spans several (request, KV head) units and cuts some of them.
    h = HeadConfig(32, 8, 128, 1e-6, 1e6)
    lens = np.random.default_rng(11).integers(0, 200, size=600).tolist()
    dec = make_decode_inputs(h, lens, seed=12, device=DEV, capacity=201)
    err = _check_decode(dec)
    note(f"600 short requests: max-abs error {err:.3e}")


def test_decode_long_requests_split_over_many_wavefronts():
    # 3 x 8 units of ~1250 steps over 2048 wavefronts: every unit is cut into
    # ~80 portions merged by the combine.
    h = HeadConfig(32, 8, 128, 1e-6, 1e6)
    dec = make_decode_inputs(h, [40000, 39999, 20001], seed=13, device=DEV, capacity=40001)
    err = _check_decode(dec)
    note(f"long requests: max-abs error {err:.3e}")


def test_decode_is_deterministic():
    h = HeadConfig(32, 8, 128, 1e-6, 1e6)
    outs = []
    for _ in range(2):
        dec = make_decode_inputs(h, [3000, 10, 700], seed=3, device=DEV)
        outs.append(run_decode(dec)["out"])
    assert torch.equal(bits(outs[0]), bits(outs[1]))


def _chained(name):
    """Prefill, then decode steps on the cache the prefill wrote, against the oracle doing the same."""
    w = build_workload(name, device=DEV)
    p = w.prefill
    h = p.heads
    run_prefill(p)
    ref = oracle_prefill(p)
    kc, vc = ref["k_cache"], ref["v_cache"]
    t = p.seqlens[0]
    errs = []
    for s, row in enumerate(w.chained_decode_qkv):
        L = t + s
        lens = torch.tensor([L], dtype=torch.int32, device=DEV)

        class Step:  # the decode arguments for this step
            heads = h
            qkv = row
            q_norm_weight = p.q_norm_weight
            k_norm_weight = p.k_norm_weight
            positions = lens.clone()
            cache_lens = lens
            cache_capacity = p.cache_capacity
            k_cache = p.k_cache
            v_cache = p.v_cache
            num_seqs = 1
            max_cache_len = L

        got = run_decode(Step)["out"]
        r = oracle.decode(f64(row), f64(p.q_norm_weight), f64(p.k_norm_weight), [L], [L], kc, vc, **layer_kw(h))
        kc, vc = r["k_cache"], r["v_cache"]
        errs.append(assert_close(f64(got), r["out"], BF16_TOL, f"{name} decode step {s}"))
        assert torch.equal(bits(p.v_cache[0, :, L]), bits(row[0, (h.num_q_heads + h.num_kv_heads) * h.head_dim:]
                                                          .reshape(h.num_kv_heads, h.head_dim)))
    note(f"{name}: chained decode max-abs errors {['%.2e' % e for e in errs]}")


def test_chained_decode_single_t64():
    _chained("single_t64_hq4_hkv2_d64")


def test_chained_decode_pages_t12_9_steps():
    _chained("pages_t12_decode9")


def test_decode_equals_last_prefill_row_on_gpu():
    # A decode step over L cached tokens and a prefill over the same L+1 tokens
    # compute the same row (different kernels, so compared to the tolerance).
    from workloads import make_prefill_inputs

    h = HeadConfig(32, 8, 128, 1e-6, 1e6)
    for L in (0, 37, 600):
        p = make_prefill_inputs(h, [L + 1], seed=L, device=DEV, capacity=L + 1)
        full = run_prefill(p)["out"]
        k = p.k_cache.clone()
        v = p.v_cache.clone()
        k[:, :, L:] = float("nan")
        v[:, :, L:] = float("nan")

        class Step:
            heads = h
            qkv = p.qkv[L:L + 1]
            q_norm_weight = p.q_norm_weight
            k_norm_weight = p.k_norm_weight
            positions = torch.tensor([L], dtype=torch.int32, device=DEV)
            cache_lens = torch.tensor([L], dtype=torch.int32, device=DEV)
            cache_capacity = L + 1
            k_cache = k
            v_cache = v
            num_seqs = 1
            max_cache_len = L

        got = run_decode(Step)["out"]
        assert_close(f64(got), f64(full[L:L + 1]), BF16_TOL, f"decode vs prefill row at L={L}")
        # The decode wrote the same K~/V the prefill wrote for that token.
        assert torch.equal(bits(v), bits(p.v_cache))
        assert torch.equal(bits(k), bits(p.k_cache))


def test_decode_qwen3_4b_64_requests_full():
    # 64 requests, cache lengths U[512, 8192], Hq=32 Hkv=8 D=128 -- the launch shape the benchmark times.
    # Every request's output row and new cache slots against the oracle.
    w = build_workload("qwen3_4b_decode64", device=DEV)
    err = _check_decode(w.decode)
    note(f"decode64: all 64 requests, max-abs error {err:.3e}")


def test_decode_mixed_step_part_full():
    # The decode half of the mixed step: 128 requests, cache lengths U[1, 16384], all checked.
    w = build_workload("mixed_qwen3_8b", device=DEV)
    err = _check_decode(w.decode)
    note(f"mixed decode: all 128 requests, max-abs error {err:.3e}")


# Units that one wavefront covers, units cut over many wavefronts, several
# query-head chunks per KV head, and idle wavefronts.
MERGE_CASES = [
    (32, 8, 128, [0, 3, 17, 31, 32, 33, 64, 150]),
    (32, 8, 128, [20000, 2, 9000]),
    (48, 3, 128, [5000, 7]),
    (10, 2, 64, [12000, 400, 0]),
]


@pytest.mark.parametrize("case", MERGE_CASES, ids=_ids)
def test_decode_writes_every_row_once_and_reuses_its_workspace(case):
    """`out` starts as NaN, so a head that the combine never stored shows.  Two calls share one workspace (the
    plan and the partial records of the first call are still there) and give the same bits."""
    import decoder_attention_amd as da
    from harness import cfg_of

    hq, hkv, d, lens = case
    h = HeadConfig(hq, hkv, d, 1e-6, 1e6)
    note(f"decode merge {_ids(case)}")
    cfg = cfg_of(h, torch.bfloat16)
    ws = None
    outs = []
    for _ in range(2):
        dec = make_decode_inputs(h, lens, seed=77, device=DEV, capacity=max(lens) + 1)
        ref = oracle.decode(f64(dec.qkv), f64(dec.q_norm_weight), f64(dec.k_norm_weight), dec.positions.cpu().numpy(),
                            np.array(lens), f64(dec.k_cache), f64(dec.v_cache), **layer_kw(h))
        out = torch.full((len(lens), hq * d), float("nan"), dtype=torch.bfloat16, device=DEV)
        out, ws = da.decode(cfg, dec.qkv, dec.q_norm_weight, dec.k_norm_weight, dec.positions, dec.cache_lens,
                            max(lens), dec.k_cache, dec.v_cache, out=out, workspace=ws)
        torch.cuda.synchronize()
        assert_close(f64(out), ref["out"], BF16_TOL, "decode out")
        outs.append(out.clone())
    assert torch.equal(bits(outs[0]), bits(outs[1]))
