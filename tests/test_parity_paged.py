"""Attention over a paged K/V cache on the GPU, through the C ABI.

A paged cache stores each request's slots in pages of a pool found through a block table; every result equals
the contiguous call's on the logical cache the table describes.  The paged kernels read the same values in the
same order as the contiguous ones, so each case is checked two ways:

* bit for bit against the contiguous call on the same logical cache (outputs and written slots);
* against the paged oracle (``oracle.paged``), which gathers through the table itself.

Tables are random permutations of the pool's pages (pages out of order, holes no request owns); the pools start
as NaN, so a read of a hole or of an unwritten slot, or a write to the wrong page, shows.  Every pool entry other
than the call's new slots must keep its bits.
"""

import numpy as np
import pytest
import torch

import decoder_attention_amd as da
import oracle
from harness import (BF16_TOL, assert_close, bits, cfg_of, f64, layer_kw, note, oracle_decode_rows, tol_for)
from workloads import (HeadConfig, build_workload, make_append_inputs, make_decode_inputs, make_prefill_inputs,
                       paged_from_contiguous)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _nan(shape, dtype):
    return torch.full(shape, float("nan"), dtype=dtype, device=DEV)


def _slot_mask(pc, lens_new):
    """Pool mask [num_pages, P] of the slots a call writes: request b's slots lens_new[b] (a list of slots)."""
    mask = torch.zeros((pc.num_pages, pc.page_size), dtype=torch.bool, device=DEV)
    tab = pc.block_table.long()
    for b, slots in enumerate(lens_new):
        for s in slots:
            mask[tab[b, s // pc.page_size], s % pc.page_size] = True
    return mask


def _pool_rows(pool, table, b, slots, page_size):
    """[len(slots), Hkv, D] rows of request b's logical cache, read through the table."""
    tab = table.long()
    return torch.stack([pool[tab[b, s // page_size], :, s % page_size] for s in slots])


def _check_untouched(pc, k0, v0, written):
    mask = _slot_mask(pc, written)[:, None, :, None].expand_as(pc.k_pool)
    assert torch.equal(bits(pc.k_pool)[~mask], bits(k0)[~mask]), "a K pool entry outside the new slots changed"
    assert torch.equal(bits(pc.v_pool)[~mask], bits(v0)[~mask]), "a V pool entry outside the new slots changed"


DECODE_CASES = [
    (32, 8, 128, [0, 1, 63, 64, 65, 700, 2047]),
    (4, 2, 64, [5, 300, 129]),
    (20, 1, 128, [250, 0, 1000]),     # G = 20: two matrix tiles of 10 query heads per KV head
]


@pytest.mark.parametrize("page_size", [64, 128, 256])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: f"hq{c[0]}-hkv{c[1]}-d{c[2]}")
def test_paged_decode(case, dtype, page_size):
    hq, hkv, d, lens = case
    h = HeadConfig(hq, hkv, d, 1e-6, 1e6)
    note(f"paged decode {hq}/{hkv}/{d} {dtype} P={page_size} lens {lens}")
    dec = make_decode_inputs(h, lens, seed=sum(lens) % 997 + page_size, dtype=dtype, device=DEV)
    pc = paged_from_contiguous(dec.k_cache, dec.v_cache, page_size, seed=page_size + 7)
    k0, v0 = pc.k_pool.clone(), pc.v_pool.clone()
    cfg = cfg_of(h, dtype)
    width = hq * d
    ref, _ = da.decode(cfg, dec.qkv, dec.q_norm_weight, dec.k_norm_weight, dec.positions, dec.cache_lens,
                       dec.max_cache_len, dec.k_cache, dec.v_cache, out=_nan((len(lens), width), dtype))
    got, _ = da.decode_paged(cfg, dec.qkv, dec.q_norm_weight, dec.k_norm_weight, dec.positions, dec.cache_lens,
                             dec.max_cache_len, pc.k_pool, pc.v_pool, pc.block_table, page_size,
                             out=_nan((len(lens), width), dtype))
    torch.cuda.synchronize()
    assert torch.equal(bits(got), bits(ref)), "paged decode differs from the contiguous decode"
    for b, L in enumerate(lens):
        assert torch.equal(bits(_pool_rows(pc.k_pool, pc.block_table, b, [L], page_size)[0]),
                           bits(dec.k_cache[b, :, L])), f"new K slot of request {b}"
        assert torch.equal(bits(_pool_rows(pc.v_pool, pc.block_table, b, [L], page_size)[0]),
                           bits(dec.v_cache[b, :, L])), f"new V slot of request {b}"
    _check_untouched(pc, k0, v0, [[L] for L in lens])
    want = oracle.paged.decode(f64(dec.qkv), f64(dec.q_norm_weight), f64(dec.k_norm_weight),
                               dec.positions.cpu().numpy(), lens, f64(k0), f64(v0), pc.block_table.cpu().numpy(),
                               page_size, **layer_kw(h))
    assert_close(f64(got), want["out"], tol_for(dtype), "paged decode out")
    new_k = torch.stack([_pool_rows(pc.k_pool, pc.block_table, b, [L], page_size)[0] for b, L in enumerate(lens)])
    assert_close(f64(new_k), want["k_tilde"], tol_for(dtype), "paged decode new K slots")


@pytest.mark.parametrize("page_size", [64, 256])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
@pytest.mark.parametrize("hq,hkv,d", [(32, 8, 128), (8, 8, 64), (16, 2, 128)], ids=["g4d128", "g1d64", "g8d128"])
def test_paged_prefill_then_append(hq, hkv, d, dtype, page_size):
    """A prefill into an empty paged cache (no history: the unshifted softmax in bf16), then a chunk appended on
    top of it (the running-max kernel), each equal to the contiguous call and to the paged oracle."""
    h = HeadConfig(hq, hkv, d, 1e-6, 1e6)
    lens = [300, 1, 0, 129]
    chunks = [70, 0, 5, 64]
    cap = max(p + c for p, c in zip(lens, chunks))
    note(f"paged prefill + append {hq}/{hkv}/{d} {dtype} P={page_size}")
    p = make_prefill_inputs(h, lens, seed=101, dtype=dtype, device=DEV, capacity=cap)
    pc = paged_from_contiguous(p.k_cache, p.v_cache, page_size, seed=page_size + 11)
    k0, v0 = pc.k_pool.clone(), pc.v_pool.clone()
    cfg = cfg_of(h, dtype)
    width = hq * d
    ref, _ = da.prefill(cfg, p.qkv, p.q_norm_weight, p.k_norm_weight, p.positions, p.cu_seqlens, p.max_seqlen,
                        p.k_cache, p.v_cache, out=_nan((p.num_tokens, width), dtype))
    got, _ = da.prefill_append_paged(cfg, p.qkv, p.q_norm_weight, p.k_norm_weight, p.positions, p.cu_seqlens, None,
                                     p.max_seqlen, 0, pc.k_pool, pc.v_pool, pc.block_table, page_size,
                                     out=_nan((p.num_tokens, width), dtype))
    torch.cuda.synchronize()
    assert torch.equal(bits(got), bits(ref)), "paged prefill differs from the contiguous prefill"
    for b, t in enumerate(lens):
        if t:
            assert torch.equal(bits(_pool_rows(pc.k_pool, pc.block_table, b, range(t), page_size)),
                               bits(p.k_cache[b, :, :t].permute(1, 0, 2))), f"K slots of request {b}"
            assert torch.equal(bits(_pool_rows(pc.v_pool, pc.block_table, b, range(t), page_size)),
                               bits(p.v_cache[b, :, :t].permute(1, 0, 2))), f"V slots of request {b}"
    _check_untouched(pc, k0, v0, [list(range(t)) for t in lens])
    want = oracle.paged.prefill_append(f64(p.qkv), f64(p.q_norm_weight), f64(p.k_norm_weight),
                                       p.positions.cpu().numpy(), p.cu_seqlens.cpu().numpy(), [0] * len(lens), f64(k0),
                                       f64(v0), pc.block_table.cpu().numpy(), page_size, **layer_kw(h))
    assert_close(f64(got), want["out"], tol_for(dtype), "paged prefill out")

    # Append a chunk per request on top of what the prefill wrote (contiguous and paged side by side).
    a = make_append_inputs(h, lens, chunks, seed=102, dtype=dtype, device=DEV, capacity=cap)
    a.q_norm_weight.copy_(p.q_norm_weight)
    a.k_norm_weight.copy_(p.k_norm_weight)
    k1, v1 = pc.k_pool.clone(), pc.v_pool.clone()
    ref2, _ = da.prefill_append(cfg, a.qkv, a.q_norm_weight, a.k_norm_weight, a.positions, a.cu_seqlens,
                                a.cache_lens, a.max_seqlen, a.max_cache_len, p.k_cache, p.v_cache,
                                out=_nan((a.num_tokens, width), dtype))
    got2, _ = da.prefill_append_paged(cfg, a.qkv, a.q_norm_weight, a.k_norm_weight, a.positions, a.cu_seqlens,
                                      a.cache_lens, a.max_seqlen, a.max_cache_len, pc.k_pool, pc.v_pool,
                                      pc.block_table, page_size, out=_nan((a.num_tokens, width), dtype))
    torch.cuda.synchronize()
    assert torch.equal(bits(got2), bits(ref2)), "paged append differs from the contiguous append"
    _check_untouched(pc, k1, v1, [list(range(P, P + c)) for P, c in zip(lens, chunks)])
    want2 = oracle.paged.prefill_append(f64(a.qkv), f64(a.q_norm_weight), f64(a.k_norm_weight),
                                        a.positions.cpu().numpy(), a.cu_seqlens.cpu().numpy(), lens, f64(k1), f64(v1),
                                        pc.block_table.cpu().numpy(), page_size, **layer_kw(h))
    assert_close(f64(got2), want2["out"], tol_for(dtype), "paged append out")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_paged_decode_shared_prefix(dtype):
    """Requests whose tables share their first two pages (a prefix stored once) all read it; their new tokens go
    to pages of their own and the shared pages are not written."""
    h = HeadConfig(32, 8, 128, 1e-6, 1e6)
    page_size = 64
    lens = [200, 128, 131, 500]                       # every history covers the two shared pages
    dec = make_decode_inputs(h, lens, seed=103, dtype=dtype, device=DEV)
    pc = paged_from_contiguous(dec.k_cache, dec.v_cache, page_size, seed=104, shared_prefix_pages=2)
    assert int(pc.block_table[:, :2].unique().numel()) == 2
    k0, v0 = pc.k_pool.clone(), pc.v_pool.clone()
    cfg = cfg_of(h, dtype)
    got, _ = da.decode_paged(cfg, dec.qkv, dec.q_norm_weight, dec.k_norm_weight, dec.positions, dec.cache_lens,
                             dec.max_cache_len, pc.k_pool, pc.v_pool, pc.block_table, page_size,
                             out=_nan((len(lens), 32 * 128), dtype))
    torch.cuda.synchronize()
    _check_untouched(pc, k0, v0, [[L] for L in lens])
    want = oracle.paged.decode(f64(dec.qkv), f64(dec.q_norm_weight), f64(dec.k_norm_weight),
                               dec.positions.cpu().numpy(), lens, f64(k0), f64(v0), pc.block_table.cpu().numpy(),
                               page_size, **layer_kw(h))
    assert_close(f64(got), want["out"], tol_for(dtype), "shared-prefix decode out")


@pytest.mark.parametrize("page_size", [64, 1024])
def test_paged_decode_benchmark_workload(page_size):
    """The mixed step's 128 decodes (cache lengths up to 16384) from a paged pool: every output and new slot
    equals the contiguous decode bit for bit, and every request against the oracle."""
    w = build_workload("mixed_qwen3_8b", device=DEV)
    dec = w.decode
    note(f"paged decode of the benchmark workload, P={page_size}")
    pc = paged_from_contiguous(dec.k_cache, dec.v_cache, page_size, seed=105)
    cfg = cfg_of(dec.heads, dec.qkv.dtype)
    k0, v0 = dec.k_cache.clone(), dec.v_cache.clone()
    ref, _ = da.decode(cfg, dec.qkv, dec.q_norm_weight, dec.k_norm_weight, dec.positions, dec.cache_lens,
                       dec.max_cache_len, dec.k_cache, dec.v_cache)
    got, _ = da.decode_paged(cfg, dec.qkv, dec.q_norm_weight, dec.k_norm_weight, dec.positions, dec.cache_lens,
                             dec.max_cache_len, pc.k_pool, pc.v_pool, pc.block_table, page_size)
    torch.cuda.synchronize()
    assert torch.equal(bits(got), bits(ref)), "paged decode differs from the contiguous decode"
    lens = dec.cache_lens.cpu().tolist()
    new_k = torch.stack([_pool_rows(pc.k_pool, pc.block_table, b, [L], page_size)[0] for b, L in enumerate(lens)])
    idx = torch.arange(len(lens), device=DEV)
    assert torch.equal(bits(new_k), bits(dec.k_cache[idx, :, dec.cache_lens.long()]))
    # Against the oracle: every request once (P = 64); the other page size equals the contiguous bits above.
    checked = None if page_size == 64 else [0, 1, 64, 127]
    want = oracle_decode_rows(dec.qkv, dec.q_norm_weight, dec.k_norm_weight, dec.positions, dec.cache_lens, k0, v0,
                              dec.heads, checked)
    sel = list(range(len(lens))) if checked is None else checked
    err = assert_close(f64(got[sel]), want["out"], BF16_TOL, f"paged decode out ({len(sel)} requests)")
    note(f"paged decode P={page_size}: max-abs error {err:.3e}")


def test_paged_append_chunked_workload_sampled():
    """2048-token chunks onto 8 histories of 2k-14k entries (the chunked-prefill workload) from a paged pool
    (P = 256): the output equals the contiguous append bit for bit, sampled rows against the oracle."""
    w = build_workload("chunked_qwen3_8b", device=DEV)
    a = w.append
    page_size = 256
    pc = paged_from_contiguous(a.k_cache, a.v_cache, page_size, seed=106)
    cfg = cfg_of(a.heads, a.qkv.dtype)
    k0, v0 = a.k_cache.clone(), a.v_cache.clone()
    note("paged append of the chunked workload, P=256")
    ref, _ = da.prefill_append(cfg, a.qkv, a.q_norm_weight, a.k_norm_weight, a.positions, a.cu_seqlens,
                               a.cache_lens, a.max_seqlen, a.max_cache_len, a.k_cache, a.v_cache)
    got, _ = da.prefill_append_paged(cfg, a.qkv, a.q_norm_weight, a.k_norm_weight, a.positions, a.cu_seqlens,
                                     a.cache_lens, a.max_seqlen, a.max_cache_len, pc.k_pool, pc.v_pool,
                                     pc.block_table, page_size)
    torch.cuda.synchronize()
    assert torch.equal(bits(got), bits(ref)), "paged append differs from the contiguous append"
    # Sampled rows of each request against the oracle's own q~/k~ over that request's cached history.
    h = a.heads
    qt, kt, v = oracle.qk_norm_rope(f64(a.qkv), f64(a.q_norm_weight), f64(a.k_norm_weight), a.positions.cpu().numpy(),
                                    **layer_kw(h))
    cu = a.cu_seqlens.cpu().tolist()
    rng = np.random.default_rng(7)
    group = h.num_q_heads // h.num_kv_heads
    for r, (past, t) in enumerate(zip(a.past_lens, a.seqlens)):
        hist_k, hist_v = f64(k0[r, :, :past]), f64(v0[r, :, :past])
        for j in sorted({0, t - 1} | set(int(x) for x in rng.choice(t, 2, replace=False))):
            n = cu[r] + j
            row = np.empty((h.num_q_heads, h.head_dim))
            for hh in range(h.num_q_heads):
                g = hh // group
                row[hh] = oracle.attend_prefix(qt[n, hh], np.concatenate([hist_k[g], kt[cu[r]:n + 1, g]]),
                                               np.concatenate([hist_v[g], v[cu[r]:n + 1, g]]))
            assert_close(f64(got[n]).reshape(row.shape), row, BF16_TOL, f"paged append row {n} of request {r}")
