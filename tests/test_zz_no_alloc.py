"""qknorm_rope_attn_decode_noalloc on the GPU: the decode entry point that allocates nothing.

It runs the same kernels as qknorm_rope_attn_decode with the workspace in the library's fixed per-GPU scratch,
so its output and caches must equal the workspace entry point's bit for bit.  Two calls in a row share the
scratch, the second with fewer requests and shorter caches than the first: what the first call left there must
not leak into the second.  Every case runs through the C ABI.
"""

import pytest
import torch

import decoder_attention_amd as da
from harness import bits, cfg_of, note
from workloads import HeadConfig, make_decode_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _pair(h, lens, seed, dtype):
    """The workspace decode and the no-allocation decode on identical inputs and caches; returns both results."""
    d = make_decode_inputs(h, lens, seed=seed, dtype=dtype, device=DEV)
    cfg = cfg_of(h, dtype)
    width = h.num_q_heads * h.head_dim
    k2, v2 = d.k_cache.clone(), d.v_cache.clone()
    ref = torch.full((d.num_seqs, width), float("nan"), dtype=dtype, device=DEV)
    da.decode(cfg, d.qkv, d.q_norm_weight, d.k_norm_weight, d.positions, d.cache_lens, d.max_cache_len,
              d.k_cache, d.v_cache, out=ref)
    got = torch.full((d.num_seqs, width), float("nan"), dtype=dtype, device=DEV)
    st = da.qknorm_rope_attn_decode_noalloc(cfg, d.qkv, d.q_norm_weight, d.k_norm_weight, d.positions,
                                            d.cache_lens, d.num_seqs, d.max_cache_len, k2, v2, d.cache_capacity,
                                            got, None)
    assert st == da.QKRA_OK, da.qknorm_rope_attn_status_string(st)
    torch.cuda.synchronize()
    return (ref, d.k_cache, d.v_cache), (got, k2, v2)


def _assert_same(a, b, what):
    for name, x, y in zip(("out", "K cache", "V cache"), a, b):
        assert torch.equal(bits(x), bits(y)), f"{what}: {name} differs from the workspace decode"
    assert torch.isfinite(b[0].float()).all(), f"{what}: unwritten output rows"


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_noalloc_decode_equals_workspace_decode_twice(dtype):
    h = HeadConfig(32, 8, 128, 1e-6, 1e6)
    first = [4000, 17, 0, 9000, 2500, 31, 33, 700]   # more requests, longer caches
    second = [5, 1200, 64]                             # then fewer and shorter, on the same scratch
    note(f"noalloc decode {dtype}: {len(first)} requests, then {len(second)}")
    a, b = _pair(h, first, 91, dtype)
    _assert_same(a, b, "first call")
    a, b = _pair(h, second, 92, dtype)
    _assert_same(a, b, "second call")


def test_noalloc_decode_other_heads_and_the_limit():
    # A grouping with two matrix tiles per KV head (G = 10 -> 5 + 5) and D = 64, then a call past the scratch.
    h = HeadConfig(20, 2, 64, 1e-6, 1e4)
    note("noalloc decode Hq 20 Hkv 2 D 64")
    a, b = _pair(h, [300, 0, 1500], 93, torch.bfloat16)
    _assert_same(a, b, "G = 10")
    big = HeadConfig(32, 8, 128, 1e-6, 1e6)
    cfg = cfg_of(big, torch.bfloat16)
    assert da.qknorm_rope_attn_workspace_bytes(cfg, da.QKRA_MODE_DECODE, 4096, 10) > da.QKRA_NOALLOC_SCRATCH_BYTES
    d = make_decode_inputs(big, [10] * 4096, seed=94, device=DEV, capacity=11)
    out = torch.empty((4096, 32 * 128), dtype=torch.bfloat16, device=DEV)
    st = da.qknorm_rope_attn_decode_noalloc(cfg, d.qkv, d.q_norm_weight, d.k_norm_weight, d.positions, d.cache_lens,
                                            4096, 10, d.k_cache, d.v_cache, 11, out, None)
    assert st == da.QKRA_ERR_SCRATCH_LIMIT
