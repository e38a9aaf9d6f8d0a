"""Prefill on the GPU, through the C ABI, against the fp64 oracle."""

import zlib

import numpy as np
import pytest
import torch

import decoder_attention_amd as da
import harness
import oracle
from harness import (BF16_TOL, FP32_TOL, assert_close, bits, check_prefill_caches, f64, layer_kw, note,
                     oracle_prefill, run_prefill, sample_tokens, tol_for)
from workloads import HeadConfig, build_workload, make_prefill_inputs, prefill_inputs_from_rows

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

# (Hq, Hkv, D, request lengths, RoPE base): every GQA packing the kernel has
# (G = 1, 2, 3, 4, 8, 16), both head dims, ragged and empty requests, lengths
# on both sides of the 32-token block and 64-key tile edges.
CASES = [
    (4, 2, 64, [64], 1e4),
    (4, 2, 64, [1], 1e4),
    (16, 8, 128, [1, 31, 32, 33, 0, 65, 130], 1e6),
    (32, 8, 128, [257, 12, 100], 1e6),
    (8, 8, 128, [200, 63], 1e4),
    (16, 2, 64, [150, 40], 1e6),
    (12, 4, 128, [70, 129], 1e6),
    (32, 4, 64, [100], 1e6),
    (48, 3, 128, [77, 2], 1e4),
    # Equal-length batches (work items in query-tile order across the requests).
    (16, 4, 128, [160, 160], 1e6),
    (8, 2, 64, [96, 96, 96], 1e4),
    # Long enough for the unmasked steps that run in groups of six before the
    # general loop: lengths on both sides of 7 and 9 tiles of 64 keys.
    (32, 8, 128, [448, 449, 511, 577], 1e6),
    (16, 16, 64, [833, 64], 1e4),
    (64, 8, 64, [700], 1e6),
]


def _ids(case):
    hq, hkv, d, lens, base = case
    return f"hq{hq}-hkv{hkv}-d{d}-T{'_'.join(map(str, lens))}"


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_prefill_matches_oracle(case, dtype):
    hq, hkv, d, lens, base = case
    h = HeadConfig(hq, hkv, d, 1e-6, base)
    p = make_prefill_inputs(h, lens, seed=zlib.crc32(_ids(case).encode()) % 10000, dtype=dtype, device=DEV,
                            capacity=max(lens) + 5)
    note(f"prefill {_ids(case)} {dtype}")
    k_before, v_before = p.k_cache.clone(), p.v_cache.clone()
    got = run_prefill(p)
    ref = oracle_prefill(p)
    tol = tol_for(dtype)
    assert_close(f64(got["out"]), ref["out"], tol, "out")
    if got["q_tilde"] is not None:  # fp32 mode keeps q~ in the workspace
        assert_close(f64(got["q_tilde"]), ref["q_tilde"], tol, "q~ in the workspace")
    check_prefill_caches(p, k_before, v_before, ref, tol)


@pytest.mark.parametrize("hq,hkv,d,length", [(32, 8, 128, 200), (16, 2, 64, 130)])
def test_item_order_leaves_results_unchanged(hq, hkv, d, length):
    """Every work item is computed the same way whatever order the grid runs them in.  An equal-length
    batch (items by query tile across the requests) and the same requests followed by a shorter one (items
    request by request) give bit-identical rows and caches for the shared requests, and both match the
    oracle."""
    h = HeadConfig(hq, hkv, d, 1e-6, 1e6)
    longer = make_prefill_inputs(h, [length] * 3 + [7], seed=4242 + d, device=DEV, capacity=length + 3)
    n = 3 * length
    equal = prefill_inputs_from_rows(h, longer.qkv[:n], longer.q_norm_weight, longer.k_norm_weight, [length] * 3,
                                     device=DEV, capacity=length + 3)
    note(f"item order hq{hq} hkv{hkv} d{d} L{length}")
    a = run_prefill(equal)["out"]
    b = run_prefill(longer)["out"]
    assert torch.equal(bits(a), bits(b[:n])), "rows differ between the two item orders"
    assert torch.equal(bits(equal.k_cache), bits(longer.k_cache[:3])), "K cache differs"
    assert torch.equal(bits(equal.v_cache), bits(longer.v_cache[:3])), "V cache differs"
    assert_close(f64(a), oracle_prefill(equal)["out"], BF16_TOL, "out")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_single_token_returns_v_exactly(dtype):
    h = HeadConfig(32, 8, 128, 1e-6, 1e6)
    p = make_prefill_inputs(h, [1, 1, 1], seed=7, dtype=dtype, device=DEV)
    got = run_prefill(p)
    v = p.qkv[:, (32 + 8) * 128:].reshape(3, 8, 128)
    out = got["out"].reshape(3, 32, 128)
    for hh in range(32):
        assert torch.equal(bits(out[:, hh].contiguous()), bits(v[:, hh // 4].contiguous()))


@pytest.mark.parametrize("d", [128, 64])
def test_bf16_workspace_holds_the_rope_table(d):
    # The documented bf16 workspace: fp32 [N][D], cos then sin, pair i of each
    # half at (D/4)*((i/4)%2) + 4*(i/8) + i%4; values are the fp64 cos/sin of
    # p * theta_i rounded to fp32 (within one fp32 ulp of the oracle's angle).
    h = HeadConfig(16, 8, d, 1e-6, 1e6)
    lens = [1, 31, 0, 65, 130]
    p = make_prefill_inputs(h, lens, seed=21, device=DEV, capacity=max(lens))
    cfg = harness.cfg_of(h, torch.bfloat16)
    _, ws = da.prefill(cfg, p.qkv, p.q_norm_weight, p.k_norm_weight, p.positions, p.cu_seqlens, p.max_seqlen,
                       p.k_cache, p.v_cache)
    torch.cuda.synchronize()
    n = p.num_tokens
    table = ws[: n * d * 4].view(torch.float32).view(n, d).cpu().numpy().astype(np.float64)
    i = np.arange(d // 2)
    at = (d // 4) * ((i // 4) % 2) + 4 * (i // 8) + i % 4
    assert sorted(at.tolist()) == list(range(d // 2))
    ang = p.positions.cpu().numpy().astype(np.float64)[:, None] * oracle.rope_frequencies(d, 1e6)[None, :]
    for got, want in ((table[:, at], np.cos(ang)), (table[:, d // 2 + at], np.sin(ang))):
        want32 = want.astype(np.float32).astype(np.float64)
        ulp = np.spacing(np.abs(want32).astype(np.float32)).astype(np.float64)
        assert (np.abs(got - want32) <= ulp).all(), f"max error {np.abs(got - want32).max():.3e}"


def test_prefill_is_deterministic_and_causal():
    h = HeadConfig(32, 8, 128, 1e-6, 1e6)
    lens = [300, 190]
    p = make_prefill_inputs(h, lens, seed=11, device=DEV)
    first = run_prefill(p)["out"].clone()
    p2 = make_prefill_inputs(h, lens, seed=11, device=DEV)
    again = run_prefill(p2)["out"]
    assert torch.equal(bits(first), bits(again)), "repeat run differs"
    # Alter every token after row i of request 0 (and all of request 1's
    # tokens after its row j); earlier rows must not change at all.
    i, j = 131, 64
    p3 = make_prefill_inputs(h, lens, seed=11, device=DEV)
    g = torch.Generator(device="cpu").manual_seed(99)
    p3.qkv[i + 1: 300] = torch.randn(p3.qkv[i + 1: 300].shape, generator=g).to(p3.qkv.dtype).to(DEV)
    p3.qkv[300 + j + 1:] = torch.randn(p3.qkv[300 + j + 1:].shape, generator=g).to(p3.qkv.dtype).to(DEV)
    changed = run_prefill(p3)["out"]
    assert torch.equal(bits(changed[: i + 1]), bits(first[: i + 1]))
    assert torch.equal(bits(changed[300: 300 + j + 1]), bits(first[300: 300 + j + 1]))
    assert not torch.equal(bits(changed[i + 1: 300]), bits(first[i + 1: 300]))


def test_prefill_pages_shapes_workload():
    # 12-token prompt on Qwen3-4B heads.
    w = build_workload("pages_t12_decode9", device=DEV)
    p = w.prefill
    k0, v0 = p.k_cache.clone(), p.v_cache.clone()
    got = run_prefill(p)
    assert tuple(got["out"].shape) == (12, 4096)
    ref = oracle_prefill(p)
    assert_close(f64(got["out"]), ref["out"], BF16_TOL, "out")
    check_prefill_caches(p, k0, v0, ref, BF16_TOL)


def test_prefill_varlen8_full():
    # Eight packed requests, lengths U[128, 2048], Hq=16 Hkv=8 D=128: every row checked.
    w = build_workload("qwen3_0p6b_prefill_varlen8", device=DEV)
    p = w.prefill
    note(f"varlen8 lengths {p.seqlens}")
    k0, v0 = p.k_cache.clone(), p.v_cache.clone()
    got = run_prefill(p)
    ref = oracle_prefill(p)
    err = assert_close(f64(got["out"]), ref["out"], BF16_TOL, "out")
    note(f"varlen8 max-abs error {err:.3e}")
    check_prefill_caches(p, k0, v0, ref, BF16_TOL)


def _sampled_prefill_check(p, per_request, seed, min_rows=0):
    k0, v0 = p.k_cache.clone(), p.v_cache.clone()
    got = run_prefill(p)
    qt, kt, v = oracle.qk_norm_rope(f64(p.qkv), f64(p.q_norm_weight), f64(p.k_norm_weight),
                                    p.positions.cpu().numpy(), **layer_kw(p.heads))
    cu = p.cu_seqlens.cpu().tolist()
    # Every cache entry: V bit-exact, K against the oracle's k~, untouched slots intact.
    check_prefill_caches(p, k0, v0, {"k_tilde": kt}, BF16_TOL)
    rows = sample_tokens(cu, per_request, seed)
    assert len(rows) >= min_rows, f"only {len(rows)} rows sampled"
    want = oracle.prefill_rows(qt, kt, v, cu, rows)
    out = got["out"].reshape(p.num_tokens, p.heads.num_q_heads, p.heads.head_dim)
    idx = torch.tensor(rows, device=out.device)
    got_rows = f64(out.index_select(0, idx))
    err = assert_close(got_rows, np.stack([want[n] for n in rows]), BF16_TOL, f"{len(rows)} sampled rows")
    note(f"sampled {len(rows)} rows x {p.heads.num_q_heads} heads, max-abs error {err:.3e}")


def test_prefill_long_32k_sampled():
    # One request of 32768 tokens, Hq=32 Hkv=8 D=128, in the launch shape the benchmark times.
    w = build_workload("long_prefill_32k", device=DEV)
    _sampled_prefill_check(w.prefill, per_request=540, seed=4, min_rows=512)  # every head of each row


def test_prefill_mixed_step_part_sampled():
    w = build_workload("mixed_qwen3_8b", device=DEV)
    _sampled_prefill_check(w.prefill, per_request=136, seed=5, min_rows=512)
