"""The seeded generators: deterministic, shaped as the layer expects, sentinel-filled caches."""

import torch

from workloads import HeadConfig, build_workload, make_decode_inputs, make_prefill_inputs, qkv_width


def test_prefill_generator_shapes_and_determinism():
    h = HeadConfig(4, 2, 16, 1e-6, 1e4)
    a = make_prefill_inputs(h, [3, 0, 7], seed=5)
    b = make_prefill_inputs(h, [3, 0, 7], seed=5)
    assert torch.equal(a.qkv.float(), b.qkv.float())
    assert a.qkv.shape == (10, qkv_width(h)) and a.qkv.dtype == torch.bfloat16
    assert a.cu_seqlens.tolist() == [0, 3, 3, 10]
    assert a.positions.tolist() == [0, 1, 2] + list(range(7))
    assert a.k_cache.shape == (3, 2, 7, 16) and torch.isnan(a.k_cache.float()).all()
    assert a.max_seqlen == 7 and a.num_tokens == 10 and a.num_seqs == 3


def test_decode_generator_fills_only_valid_slots():
    h = HeadConfig(4, 2, 8, 1e-6, 1e4)
    d = make_decode_inputs(h, [0, 3, 5], seed=9, dtype=torch.float32)
    assert d.k_cache.shape == (3, 2, 6, 8)
    for b, L in enumerate([0, 3, 5]):
        assert not torch.isnan(d.k_cache[b, :, :L]).any()
        assert torch.isnan(d.k_cache[b, :, L:]).all() and torch.isnan(d.v_cache[b, :, L:]).all()
    assert d.positions.tolist() == [0, 3, 5]
    z = make_decode_inputs(h, [2], seed=9, parity=False)
    assert (z.k_cache[0, :, 2:].float() == 0).all()


def test_named_small_workloads():
    w = build_workload("single_t64_hq4_hkv2_d64")
    assert w.prefill.qkv.shape == (64, (4 + 4) * 64) and len(w.chained_decode_qkv) == 1
    assert w.prefill.heads.rope_base == 1e4
    w = build_workload("pages_t12_decode9")
    assert w.prefill.seqlens == [12] and len(w.chained_decode_qkv) == 9
    w = build_workload("qwen3_0p6b_prefill_varlen8")
    assert len(w.prefill.seqlens) == 8 and all(128 <= t <= 2048 for t in w.prefill.seqlens)


def test_append_generator_positions_and_cache():
    from workloads import make_append_inputs
    h = HeadConfig(4, 2, 8, 1e-6, 1e4)
    a = make_append_inputs(h, [0, 3, 5], [2, 0, 4], seed=11, dtype=torch.float32)
    assert a.qkv.shape == (6, qkv_width(h))
    assert a.cu_seqlens.tolist() == [0, 2, 2, 6]
    assert a.positions.tolist() == [0, 1, 5, 6, 7, 8]
    assert a.cache_capacity == 9 and a.k_cache.shape == (3, 2, 9, 8)  # max P + max T
    for b, p in enumerate([0, 3, 5]):
        assert not torch.isnan(a.k_cache[b, :, :p]).any()
        assert torch.isnan(a.k_cache[b, :, p:]).all() and torch.isnan(a.v_cache[b, :, p:]).all()
    assert a.max_cache_len == 5 and a.max_seqlen == 4 and a.num_tokens == 6


def test_chunked_workload_shape():
    from workloads import WORKLOADS
    assert "chunked_qwen3_8b" in WORKLOADS


def test_norm_and_next_token_generators():
    from workloads import make_next_token_inputs, make_norm_inputs

    a = make_norm_inputs(5, 16, seed=3)
    b = make_norm_inputs(5, 16, seed=3)
    assert torch.equal(a.x, b.x) and torch.equal(a.residual, b.residual) and torch.equal(a.weight, b.weight)
    first = make_norm_inputs(5, 16, seed=3, has_residual=False)
    assert first.residual is None and not first.has_residual and torch.equal(first.x, a.x)
    nt = make_next_token_inputs([3, 0, 2], 8, 11, seed=4)
    assert nt.cu_seqlens.tolist() == [0, 3, 3, 5]
    assert nt.hidden.shape == (5, 8) and nt.logits.shape == (3, 11)


def test_layer_step_workloads_present():
    from workloads import WORKLOADS

    assert {"residual_rmsnorm_qwen3_8b", "next_token_qwen3_8b"} <= set(WORKLOADS)


def test_prefill_half_workload_shape():
    w = build_workload("prefill_4x4096_qwen3_8b", parity=False)
    p = w.prefill
    assert w.decode is None and p.seqlens == [4096] * 4 and p.max_seqlen == 4096
    assert p.qkv.shape == (4 * 4096, (32 + 2 * 8) * 128)
    assert p.positions[:4096].tolist() == list(range(4096))
