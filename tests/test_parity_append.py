"""Chunks appended to filled caches, on the GPU through the C ABI, against the fp64 oracle."""

import zlib

import numpy as np
import pytest
import torch

import decoder_attention_amd as da
import oracle
from harness import BF16_TOL, assert_close, bits, cfg_of, f64, layer_kw, note, oracle_prefill, run_prefill, tol_for
from workloads import HeadConfig, build_workload, make_append_inputs, make_prefill_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def run_append(a):
    """`out` starts as NaN, so a row that no kernel wrote fails the comparison."""
    cfg = cfg_of(a.heads, a.qkv.dtype)
    h = a.heads
    out = torch.full((a.num_tokens, h.num_q_heads * h.head_dim), float("nan"), dtype=a.qkv.dtype, device=DEV)
    out, ws = da.prefill_append(cfg, a.qkv, a.q_norm_weight, a.k_norm_weight, a.positions, a.cu_seqlens,
                                a.cache_lens, a.max_seqlen, a.max_cache_len, a.k_cache, a.v_cache, out=out)
    torch.cuda.synchronize()
    return out


def _check_caches(a, k0, v0, k_tilde, tol):
    """New slots P_r..P_r+T_r-1: V bit-exact, K against the oracle's k~; every other slot keeps its bits."""
    h = a.heads
    cu = a.cu_seqlens.cpu().tolist()
    v_new = a.qkv[:, (h.num_q_heads + h.num_kv_heads) * h.head_dim:].reshape(-1, h.num_kv_heads, h.head_dim)
    written = torch.zeros(a.k_cache.shape[:3], dtype=torch.bool, device=a.k_cache.device)
    for r, (p, t) in enumerate(zip(a.past_lens, a.seqlens)):
        if t == 0:
            continue
        lo, hi = cu[r], cu[r + 1]
        assert torch.equal(bits(a.v_cache[r, :, p:p + t]), bits(v_new[lo:hi].transpose(0, 1))), f"V slots of {r}"
        assert_close(f64(a.k_cache[r, :, p:p + t].transpose(0, 1)), k_tilde[lo:hi], tol, f"K slots of {r}")
        written[r, :, p:p + t] = True
    keep = ~written
    assert torch.equal(bits(a.k_cache)[keep], bits(k0)[keep]) and torch.equal(bits(a.v_cache)[keep], bits(v0)[keep]), \
        "a slot outside P_r..P_r+T_r-1 changed"


def _check_append(a, tol=None):
    tol = tol if tol is not None else tol_for(a.qkv.dtype)
    k0, v0 = a.k_cache.clone(), a.v_cache.clone()
    got = run_append(a)
    ref = oracle.prefill_append(f64(a.qkv), f64(a.q_norm_weight), f64(a.k_norm_weight), a.positions.cpu().numpy(),
                                a.cu_seqlens.cpu().numpy(), a.past_lens, f64(k0), f64(v0), **layer_kw(a.heads))
    err = assert_close(f64(got), ref["out"], tol, "append out")
    _check_caches(a, k0, v0, ref["k_tilde"], tol)
    return err


# (Hq, Hkv, D, cached entries P_r, chunk lengths T_r): empty and long
# histories, one-token chunks, zero-length chunks, tile and split edges,
# every query-head grouping of the prefill kernel.
CASES = [
    (4, 2, 64, [0, 5, 64], [7, 1, 30]),
    (32, 8, 128, [100, 0, 1, 63, 64, 65], [1, 64, 100, 33, 2, 130]),
    (16, 2, 128, [500, 17], [200, 0]),
    (12, 4, 64, [31, 1000], [65, 9]),
    (48, 3, 128, [64, 200], [64, 64]),
    (8, 8, 128, [10], [300]),
    # Histories that put the first masked tile just before, at and after the
    # end of a group of six unmasked steps.
    (32, 8, 128, [447, 446, 767, 383], [64, 64, 1, 130]),
]


def _ids(case):
    hq, hkv, d, past, chunks = case
    return f"hq{hq}-hkv{hkv}-d{d}-P{'_'.join(map(str, past))}-T{'_'.join(map(str, chunks))}"


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_append_matches_oracle(case, dtype):
    hq, hkv, d, past, chunks = case
    h = HeadConfig(hq, hkv, d, 1e-6, 1e6)
    note(f"append {_ids(case)} {dtype}")
    a = make_append_inputs(h, past, chunks, seed=zlib.crc32(_ids(case).encode()) % 10000, dtype=dtype, device=DEV,
                           capacity=max(past) + max(chunks) + 3)
    _check_append(a)


def test_append_to_empty_caches_equals_prefill_bitwise():
    # With every P_r = 0 the append runs the prefill's kernels on the same inputs.
    h = HeadConfig(32, 8, 128, 1e-6, 1e6)
    seqlens = [100, 1, 257]
    p = make_prefill_inputs(h, seqlens, seed=70, device=DEV, capacity=260)
    a = make_append_inputs(h, [0, 0, 0], seqlens, seed=71, device=DEV, capacity=260)
    a.qkv.copy_(p.qkv)
    a.q_norm_weight.copy_(p.q_norm_weight)
    a.k_norm_weight.copy_(p.k_norm_weight)
    want = run_prefill(p)["out"]
    got = run_append(a)
    assert torch.equal(bits(got), bits(want))
    assert torch.equal(bits(a.k_cache), bits(p.k_cache)) and torch.equal(bits(a.v_cache), bits(p.v_cache))


def test_prefill_then_append_equals_one_prefill():
    # GPU prefill of the first T1 tokens, then the next T2 appended to the cache
    # it wrote, against the oracle's prefill of all T1 + T2 tokens.
    h = HeadConfig(16, 8, 128, 1e-6, 1e6)
    splits = [(130, 70), (1, 200), (64, 1), (0, 33)]
    full = [t1 + t2 for t1, t2 in splits]
    # The append's bound on the capacity: max_r P_r + max_r T_r.
    cap = max(t1 for t1, _ in splits) + max(t2 for _, t2 in splits) + 1
    whole = make_prefill_inputs(h, full, seed=72, device=DEV, capacity=cap)
    ref = oracle_prefill(whole)
    cu = whole.cu_seqlens.cpu().tolist()
    first_rows = torch.cat([torch.arange(cu[r], cu[r] + t1) for r, (t1, _) in enumerate(splits)]).to(DEV)
    second_rows = torch.cat([torch.arange(cu[r] + t1, cu[r + 1]) for r, (t1, _) in enumerate(splits)]).to(DEV)
    pre = make_prefill_inputs(h, [t1 for t1, _ in splits], seed=73, device=DEV, capacity=cap)
    pre.qkv.copy_(whole.qkv.index_select(0, first_rows))
    pre.q_norm_weight.copy_(whole.q_norm_weight)
    pre.k_norm_weight.copy_(whole.k_norm_weight)
    run_prefill(pre)
    app = make_append_inputs(h, [t1 for t1, _ in splits], [t2 for _, t2 in splits], seed=74, device=DEV,
                             capacity=cap)
    app.qkv.copy_(whole.qkv.index_select(0, second_rows))
    app.q_norm_weight.copy_(whole.q_norm_weight)
    app.k_norm_weight.copy_(whole.k_norm_weight)
    app.k_cache.copy_(pre.k_cache)
    app.v_cache.copy_(pre.v_cache)
    got = run_append(app)
    want = ref["out"][second_rows.cpu().numpy()]
    err = assert_close(f64(got), want, BF16_TOL, "appended rows")
    for r, n in enumerate(full):
        assert torch.equal(bits(app.v_cache[r, :, :n]), bits(whole.v_cache.new_tensor(ref["v_cache"][r, :, :n])))
        assert_close(f64(app.k_cache[r, :, :n]), ref["k_cache"][r, :, :n], BF16_TOL, f"K cache of request {r}")
    note(f"prefill + append vs one prefill: max-abs error {err:.3e}")


def test_append_chunked_workload_sampled():
    # The benchmark's shape: 2048-token chunks onto 8 caches of 2048..14336
    # entries; rows sampled per request (first, last and random), each
    # against the oracle's own q~/k~ over the request's cached history.
    w = build_workload("chunked_qwen3_8b", device=DEV)
    a = w.append
    h = a.heads
    k0, v0 = a.k_cache.clone(), a.v_cache.clone()
    got = run_append(a)
    qt, kt, v = oracle.qk_norm_rope(f64(a.qkv), f64(a.q_norm_weight), f64(a.k_norm_weight), a.positions.cpu().numpy(),
                                    **layer_kw(h))
    cu = a.cu_seqlens.cpu().tolist()
    rng = np.random.default_rng(6)
    group = h.num_q_heads // h.num_kv_heads
    worst = 0.0
    for r, (past, t) in enumerate(zip(a.past_lens, a.seqlens)):
        js = sorted({0, t - 1} | set(int(x) for x in rng.choice(t, 2, replace=False)))
        hist_k = f64(k0[r, :, :past])
        hist_v = f64(v0[r, :, :past])
        for j in js:
            n = cu[r] + j
            row = np.empty((h.num_q_heads, h.head_dim))
            for hh in range(h.num_q_heads):
                g = hh // group
                keys = np.concatenate([hist_k[g], kt[cu[r]:n + 1, g]])
                vals = np.concatenate([hist_v[g], v[cu[r]:n + 1, g]])
                row[hh] = oracle.attend_prefix(qt[n, hh], keys, vals)
            worst = max(worst, assert_close(f64(got[n]).reshape(row.shape), row, BF16_TOL, f"row {n} of request {r}"))
    _check_caches(a, k0, v0, kt, BF16_TOL)
    note(f"chunked workload: sampled rows max-abs error {worst:.3e}")
