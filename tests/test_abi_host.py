"""The C ABI on the host: exported symbols, status strings, workspace sizes and
argument checks.  Every call here is rejected (or is a no-op) before any HIP
work is enqueued, so these run without a GPU; the pointers are placeholders
that are never dereferenced."""

import ctypes
import pathlib
import re

import pytest
import torch

import decoder_attention_amd as da

HEADER = pathlib.Path(__file__).resolve().parents[1] / "include" / "qknorm_rope_attn.h"


def declared_symbols():
    text = HEADER.read_text()
    return sorted(set(re.findall(r"QKRA_API\s+[\w\s\*]*?\b(qknorm_rope_attn_\w+)\s*\(", text)))


def test_header_declares_the_two_entry_points():
    names = declared_symbols()
    assert "qknorm_rope_attn_prefill" in names and "qknorm_rope_attn_decode" in names
    assert len(names) >= 8


def test_library_exports_every_declared_symbol():
    lib = da.lib()
    for name in declared_symbols():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value
    assert sorted(da.exported_symbols()) == declared_symbols()


def test_calibration_library_exports_every_declared_symbol():
    # The benchmark's roofline calibration kernels live in a library of their own (include/qkra_calibrate.h).
    text = (HEADER.parent / "qkra_calibrate.h").read_text()
    names = sorted(set(re.findall(r"QKRA_CALIB_API\s+[\w\s\*]*?\b(qkra_calibrate_\w+)\s*\(", text)))
    assert names == da.calibration_symbols() and len(names) == 4
    lib = da.calibration_lib()
    for name in names:
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value
    assert da.qkra_calibrate_mfma_flop(10, 512) == 10 * 512 * 4 * 4 * 32768
    assert da.qkra_calibrate_stream_read(None, 16, BASE, 8, 0) == 1   # refused before any launch
    assert da.qkra_calibrate_stream_read(BASE, 17, BASE, 8, 0) == 1
    assert da.qkra_calibrate_mfma_bf16(0, BASE, 8, 0) == 1
    assert da.qkra_calibrate_stream_copy(BASE, BASE + 32, 64, 0) == 1   # overlapping
    assert da.qkra_calibrate_stream_copy(BASE, None, 64, 0) == 1
    assert da.qkra_calibrate_stream_copy(BASE, BASE + 64, 17, 0) == 1


def test_status_strings_and_version():
    for code in range(8):
        assert da.qknorm_rope_attn_status_string(code)
    assert da.qknorm_rope_attn_status_string(99) == "unknown status"
    assert da.qknorm_rope_attn_version() == 400  # 0.4.0: paged caches, the caller's weight bound
    assert da.qknorm_rope_attn_last_hip_error() == 0
    assert da.qknorm_rope_attn_kernel_name(1) == "prefill_attn_mfma_bf16"
    assert da.qknorm_rope_attn_kernel_name(10) == "prefill_attn_mfma_bf16_shifted"


def test_workspace_bytes():
    cfg = da.make_config(32, 8, 128, da.QKRA_BF16)
    up = lambda n: -(-n // 256) * 256
    # bf16 prefill: the per-token RoPE table [N, D] fp32 (cos then sin), rounded up to 256 bytes
    assert da.qknorm_rope_attn_workspace_bytes(cfg, da.QKRA_MODE_PREFILL, 100, 100) == up(100 * 128 * 4)
    assert da.qknorm_rope_attn_workspace_bytes(cfg, da.QKRA_MODE_PREFILL, 1, 1) == 512
    # fp32 prefill: q~ [N, Hq, D] fp32
    assert da.qknorm_rope_attn_workspace_bytes(da.make_config(32, 8, 128, da.QKRA_FP32), da.QKRA_MODE_PREFILL,
                                               100, 100) == 100 * 32 * 128 * 4
    # bf16 decode: q~, then the int32 step plan [T, per, S0[0..N], first[0..W)]
    # over N = b * Hkv units (G = 4 heads per tile), then fp32 records
    # (m, l, pad, pad, o[D]) for N + W (unit, wavefront) slots of 4 heads.
    b, L, W = 3, 2047, 768
    n_units = b * 8
    q_bytes = up(b * 32 * 128 * 2)
    plan_bytes = up((3 + n_units + W) * 4)
    rec_bytes = up((n_units + W) * 4 * 132 * 4)
    assert da.qknorm_rope_attn_workspace_bytes(cfg, da.QKRA_MODE_DECODE, b, L) == q_bytes + plan_bytes + rec_bytes
    # fp32 decode: q~ then fp32 (m, l, o[D]) per (request, head, 1024-key split)
    cfg32 = da.make_config(32, 8, 128, da.QKRA_FP32)
    splits = (L + 1 + 1023) // 1024
    assert da.qknorm_rope_attn_workspace_bytes(cfg32, da.QKRA_MODE_DECODE, b, L) == \
        up(b * 32 * 128 * 4) + up(b * 32 * splits * 130 * 4)
    # a group of 12 heads runs as one tile of 12 columns; 48 heads over 3 KV heads: 16 per tile
    cfg12 = da.make_config(12, 1, 64, da.QKRA_BF16)
    assert da.qknorm_rope_attn_workspace_bytes(cfg12, da.QKRA_MODE_DECODE, 2, 10) == \
        up(2 * 12 * 64 * 2) + up((3 + 2 + W) * 4) + up((2 + W) * 12 * 68 * 4)
    bad = da.make_config(5, 2, 128)
    assert da.qknorm_rope_attn_workspace_bytes(bad, da.QKRA_MODE_PREFILL, 10, 10) == 0
    assert da.qknorm_rope_attn_workspace_bytes(cfg, 7, 10, 10) == 0


BASE = 1 << 32
MB = 1 << 20


def prefill_args(**over):
    cfg = over.pop("cfg", da.make_config(4, 2, 64, da.QKRA_BF16, 1e-6, 1e4))
    a = dict(qkv=BASE, q_norm_weight=BASE + 64 * MB, k_norm_weight=BASE + 65 * MB, positions=BASE + 66 * MB,
             cu_seqlens=BASE + 67 * MB, num_tokens=64, num_seqs=1, max_seqlen=64, k_cache=BASE + 100 * MB,
             v_cache=BASE + 200 * MB, cache_capacity=64, out=BASE + 300 * MB, workspace=BASE + 400 * MB,
             workspace_bytes=1 << 20, stream=0)
    a.update(over)
    return cfg, a


def call_prefill(cfg, a):
    return da.qknorm_rope_attn_prefill(cfg, a["qkv"], a["q_norm_weight"], a["k_norm_weight"], a["positions"],
                                       a["cu_seqlens"], a["num_tokens"], a["num_seqs"], a["max_seqlen"],
                                       a["k_cache"], a["v_cache"], a["cache_capacity"], a["out"], a["workspace"],
                                       a["workspace_bytes"], a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(cfg=da.make_config(5, 2, 64)), da.QKRA_ERR_INVALID_ARGUMENT),          # Hq % Hkv != 0
    (dict(cfg=da.make_config(4, 0, 64)), da.QKRA_ERR_INVALID_ARGUMENT),
    (dict(cfg=da.make_config(4, 2, 96)), da.QKRA_ERR_UNSUPPORTED),               # head_dim
    (dict(cfg=da.make_config(4, 2, 64, 7)), da.QKRA_ERR_UNSUPPORTED),            # dtype
    (dict(cfg=da.make_config(4, 2, 64, 0, -1.0)), da.QKRA_ERR_INVALID_ARGUMENT),  # eps < 0
    (dict(cfg=da.make_config(4, 2, 64, 0, 1e-6, 0.0)), da.QKRA_ERR_INVALID_ARGUMENT),  # base <= 0
    (dict(num_tokens=-1), da.QKRA_ERR_INVALID_ARGUMENT),
    (dict(max_seqlen=65), da.QKRA_ERR_INVALID_ARGUMENT),                        # longer than N
    (dict(num_tokens=64, num_seqs=2, max_seqlen=16), da.QKRA_ERR_INVALID_ARGUMENT),  # B * max < N
    (dict(num_seqs=0), da.QKRA_ERR_INVALID_ARGUMENT),
    (dict(cache_capacity=63), da.QKRA_ERR_CAPACITY),
    (dict(qkv=None), da.QKRA_ERR_INVALID_ARGUMENT),
    (dict(cu_seqlens=None), da.QKRA_ERR_INVALID_ARGUMENT),
    (dict(workspace_bytes=64 * 64 * 4 - 1), da.QKRA_ERR_WORKSPACE_TOO_SMALL),    # bf16: RoPE table [N, D] fp32
    (dict(workspace=None), da.QKRA_ERR_INVALID_ARGUMENT),
    (dict(out=BASE + 8), da.QKRA_ERR_INVALID_ARGUMENT),                          # misaligned
    (dict(out=BASE), da.QKRA_ERR_ALIASING),                                      # out over qkv
    (dict(v_cache=BASE + 100 * MB + 4096), da.QKRA_ERR_ALIASING),                # caches overlap
    (dict(workspace=BASE + 300 * MB + 256), da.QKRA_ERR_ALIASING),               # workspace over out
    (dict(k_cache=BASE + 64 * MB), da.QKRA_ERR_ALIASING),                        # cache over a weight
])
def test_prefill_argument_checks(over, status):
    cfg, a = prefill_args(**over)
    assert call_prefill(cfg, a) == status
    assert da.qknorm_rope_attn_last_hip_error() == 0  # rejected before any launch


def test_prefill_empty_batch_is_noop():
    cfg, a = prefill_args(num_tokens=0, num_seqs=0, max_seqlen=0, qkv=None, out=None, workspace=None,
                          workspace_bytes=0)
    assert call_prefill(cfg, a) == da.QKRA_OK


def decode_args(**over):
    cfg = over.pop("cfg", da.make_config(32, 8, 128, da.QKRA_BF16))
    a = dict(qkv=BASE, q_norm_weight=BASE + 64 * MB, k_norm_weight=BASE + 65 * MB, positions=BASE + 66 * MB,
             cache_lens=BASE + 67 * MB, num_seqs=4, max_cache_len=100, k_cache=BASE + 100 * MB,
             v_cache=BASE + 200 * MB, cache_capacity=101, out=BASE + 300 * MB, workspace=BASE + 400 * MB,
             workspace_bytes=16 * MB, stream=0)
    a.update(over)
    return cfg, a


def call_decode(cfg, a):
    return da.qknorm_rope_attn_decode(cfg, a["qkv"], a["q_norm_weight"], a["k_norm_weight"], a["positions"],
                                      a["cache_lens"], a["num_seqs"], a["max_cache_len"], a["k_cache"],
                                      a["v_cache"], a["cache_capacity"], a["out"], a["workspace"],
                                      a["workspace_bytes"], a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(cfg=da.make_config(32, 7, 128)), da.QKRA_ERR_INVALID_ARGUMENT),
    (dict(cfg=da.make_config(32, 8, 256)), da.QKRA_ERR_UNSUPPORTED),
    (dict(num_seqs=-2), da.QKRA_ERR_INVALID_ARGUMENT),
    (dict(max_cache_len=-1), da.QKRA_ERR_INVALID_ARGUMENT),
    (dict(cache_capacity=100), da.QKRA_ERR_CAPACITY),                            # no room for the new token
    (dict(cache_lens=None), da.QKRA_ERR_INVALID_ARGUMENT),
    (dict(workspace_bytes=1024), da.QKRA_ERR_WORKSPACE_TOO_SMALL),
    (dict(k_cache=BASE + 16 * 1024), da.QKRA_ERR_ALIASING),                     # cache over qkv [B, 48*128] bf16
    (dict(out=BASE + 200 * MB + 4096), da.QKRA_ERR_ALIASING),                    # out over the V cache
    (dict(workspace=BASE + 67 * MB), da.QKRA_ERR_ALIASING),                      # workspace over cache_lens
    # bf16 step plan counts in int32: 4096 * 8 units of 2^21 / 32 steps = 2^31
    (dict(num_seqs=4096, cache_capacity=1 << 21), da.QKRA_ERR_UNSUPPORTED),
])
def test_decode_argument_checks(over, status):
    cfg, a = decode_args(**over)
    assert call_decode(cfg, a) == status
    assert da.qknorm_rope_attn_last_hip_error() == 0  # rejected before any launch


def test_decode_empty_batch_is_noop():
    cfg, a = decode_args(num_seqs=0, qkv=None, out=None, workspace=None, workspace_bytes=0)
    assert call_decode(cfg, a) == da.QKRA_OK


def append_args(**over):
    cfg = over.pop("cfg", da.make_config(32, 8, 128, da.QKRA_BF16))
    a = dict(qkv=BASE, q_norm_weight=BASE + 64 * MB, k_norm_weight=BASE + 65 * MB, positions=BASE + 66 * MB,
             cu_seqlens=BASE + 67 * MB, cache_lens=BASE + 68 * MB, num_tokens=100, num_seqs=4, max_seqlen=40,
             max_cache_len=60, k_cache=BASE + 100 * MB, v_cache=BASE + 200 * MB, cache_capacity=100,
             out=BASE + 300 * MB, workspace=BASE + 400 * MB, workspace_bytes=16 * MB, stream=0)
    a.update(over)
    return cfg, a


def call_append(cfg, a):
    return da.qknorm_rope_attn_prefill_append(cfg, a["qkv"], a["q_norm_weight"], a["k_norm_weight"],
                                              a["positions"], a["cu_seqlens"], a["cache_lens"], a["num_tokens"],
                                              a["num_seqs"], a["max_seqlen"], a["max_cache_len"], a["k_cache"],
                                              a["v_cache"], a["cache_capacity"], a["out"], a["workspace"],
                                              a["workspace_bytes"], a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(cache_lens=None), da.QKRA_ERR_INVALID_ARGUMENT),
    (dict(max_cache_len=-1), da.QKRA_ERR_INVALID_ARGUMENT),
    (dict(cache_capacity=99), da.QKRA_ERR_CAPACITY),                             # 60 cached + 40 new > 99
    (dict(cfg=da.make_config(32, 8, 96)), da.QKRA_ERR_UNSUPPORTED),
    (dict(workspace_bytes=1024), da.QKRA_ERR_WORKSPACE_TOO_SMALL),
    (dict(cache_lens=BASE + 100 * MB + 64), da.QKRA_ERR_ALIASING),                # lengths inside the K cache
    (dict(out=BASE + 68 * MB - 64), da.QKRA_ERR_ALIASING),                        # out over cache_lens
])
def test_append_argument_checks(over, status):
    cfg, a = append_args(**over)
    assert call_append(cfg, a) == status
    assert da.qknorm_rope_attn_last_hip_error() == 0  # rejected before any launch


def test_append_empty_batch_is_noop():
    cfg, a = append_args(num_tokens=0, num_seqs=0, max_seqlen=0, qkv=None, out=None, workspace=None,
                         workspace_bytes=0, cache_lens=None)
    assert call_append(cfg, a) == da.QKRA_OK


def on_own_thread(fn):
    """Runs fn on a thread of its own and returns its result: a HIP error it records stays in that thread's
    last-error slot, which the other tests read as 'nothing was launched'."""
    import threading

    box = {}

    def run():
        try:
            box["value"] = fn()
        except BaseException as e:  # re-raised on the calling thread
            box["error"] = e

    t = threading.Thread(target=run)
    t.start()
    t.join()
    if "error" in box:
        raise box["error"]
    return box["value"]


def test_kernel_timing_toggle_without_launches():
    # Switching timing on creates the event pool (no call creates events); without a GPU that fails cleanly.
    def toggle():
        st = da.qknorm_rope_attn_set_kernel_timing(True)
        assert st in (da.QKRA_OK, da.QKRA_ERR_HIP)
        if st == da.QKRA_OK:
            assert da.qknorm_rope_attn_read_kernel_timing() == {}
        assert da.qknorm_rope_attn_set_kernel_timing(False) == 0

    on_own_thread(toggle)


# ---- steps next to the attention layer ------------------------------------------

def norm_args(**over):
    a = dict(dtype=da.QKRA_BF16, eps=1e-6, x=BASE, residual=BASE + 64 * MB, has_residual=True,
             weight=BASE + 128 * MB, out=BASE + 192 * MB, num_tokens=100, hidden_size=4096, stream=0)
    a.update(over)
    return a


def call_norm(a):
    return da.qknorm_rope_attn_fused_add_rmsnorm(a["dtype"], a["eps"], a["x"], a["residual"], a["has_residual"],
                                                 a["weight"], a["out"], a["num_tokens"], a["hidden_size"],
                                                 a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(dtype=7), da.QKRA_ERR_UNSUPPORTED),
    (dict(eps=-1.0), da.QKRA_ERR_INVALID_ARGUMENT),
    (dict(eps=float("nan")), da.QKRA_ERR_INVALID_ARGUMENT),
    (dict(hidden_size=4100), da.QKRA_ERR_INVALID_ARGUMENT),                 # not a multiple of 8
    (dict(hidden_size=0), da.QKRA_ERR_INVALID_ARGUMENT),
    (dict(hidden_size=32776), da.QKRA_ERR_UNSUPPORTED),                     # above 32768
    (dict(num_tokens=-1), da.QKRA_ERR_INVALID_ARGUMENT),
    (dict(weight=None), da.QKRA_ERR_INVALID_ARGUMENT),
    (dict(out=BASE + 192 * MB + 8), da.QKRA_ERR_INVALID_ARGUMENT),          # misaligned
    (dict(out=BASE + 4096), da.QKRA_ERR_ALIASING),                          # partly over x
    (dict(out=BASE + 64 * MB), da.QKRA_ERR_ALIASING),                       # out is the residual
    (dict(residual=BASE), da.QKRA_ERR_ALIASING),                            # residual is x, but it is read
    (dict(weight=BASE + 64 * MB + 1024), da.QKRA_ERR_ALIASING),             # weight inside the residual
])
def test_fused_add_rmsnorm_argument_checks(over, status):
    assert call_norm(norm_args(**over)) == status
    assert da.qknorm_rope_attn_last_hip_error() == 0


def test_fused_add_rmsnorm_empty_batch_is_noop():
    assert call_norm(norm_args(num_tokens=0, x=None, residual=None, weight=None, out=None)) == da.QKRA_OK


def gather_args(**over):
    a = dict(dtype=da.QKRA_BF16, hidden=BASE, cu_seqlens=BASE + 64 * MB, num_tokens=100, num_seqs=4,
             hidden_size=4096, out=BASE + 128 * MB, stream=0)
    a.update(over)
    return a


def call_gather(a):
    return da.qknorm_rope_attn_gather_last(a["dtype"], a["hidden"], a["cu_seqlens"], a["num_tokens"], a["num_seqs"],
                                           a["hidden_size"], a["out"], a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(dtype=2), da.QKRA_ERR_UNSUPPORTED),
    (dict(hidden_size=4), da.QKRA_ERR_INVALID_ARGUMENT),                    # 8 bytes: not a 16-byte multiple
    (dict(num_seqs=-1), da.QKRA_ERR_INVALID_ARGUMENT),
    (dict(cu_seqlens=None), da.QKRA_ERR_INVALID_ARGUMENT),
    (dict(out=BASE + 128 * MB + 4), da.QKRA_ERR_INVALID_ARGUMENT),          # misaligned
    (dict(out=BASE + 8192), da.QKRA_ERR_ALIASING),                          # inside hidden
    (dict(out=BASE + 64 * MB - 16), da.QKRA_ERR_ALIASING),                  # over cu_seqlens
])
def test_gather_last_argument_checks(over, status):
    assert call_gather(gather_args(**over)) == status
    assert da.qknorm_rope_attn_last_hip_error() == 0


def test_gather_last_empty_batch_is_noop():
    assert call_gather(gather_args(num_seqs=0, hidden=None, cu_seqlens=None, out=None)) == da.QKRA_OK


def argmax_args(**over):
    a = dict(dtype=da.QKRA_BF16, logits=BASE, num_rows=132, vocab=151936, row_stride=151936,
             out_index=BASE + 128 * MB, workspace=BASE + 192 * MB, workspace_bytes=1 * MB, stream=0)
    a.update(over)
    return a


def call_argmax(a):
    return da.qknorm_rope_attn_argmax(a["dtype"], a["logits"], a["num_rows"], a["vocab"], a["row_stride"],
                                      a["out_index"], a["workspace"], a["workspace_bytes"], a["stream"])


def test_argmax_workspace_bytes():
    # (value, index) records for each (row, segment): 8 segments of 132 rows of 151936.
    assert da.qknorm_rope_attn_argmax_workspace_bytes(132, 151936) == 2 * 4352
    assert da.qknorm_rope_attn_argmax_workspace_bytes(0, 10) == 0
    assert da.qknorm_rope_attn_argmax_workspace_bytes(4, 0) == 0
    for rows, vocab in ((1, 1), (1, 151936), (5000, 32000), (132, 2 ** 31 - 1)):
        assert da.qknorm_rope_attn_argmax_workspace_bytes(rows, vocab) >= rows * 8


@pytest.mark.parametrize("over,status", [
    (dict(dtype=3), da.QKRA_ERR_UNSUPPORTED),
    (dict(vocab=0), da.QKRA_ERR_INVALID_ARGUMENT),
    (dict(row_stride=151935), da.QKRA_ERR_INVALID_ARGUMENT),               # shorter than a row
    (dict(row_stride=151940), da.QKRA_ERR_INVALID_ARGUMENT),               # not a multiple of 8
    (dict(out_index=None), da.QKRA_ERR_INVALID_ARGUMENT),
    (dict(workspace_bytes=100), da.QKRA_ERR_WORKSPACE_TOO_SMALL),
    (dict(logits=BASE + 2), da.QKRA_ERR_INVALID_ARGUMENT),                  # misaligned
    (dict(out_index=BASE + 1024), da.QKRA_ERR_ALIASING),                    # inside the logits
    (dict(workspace=BASE + 38 * MB), da.QKRA_ERR_ALIASING),                 # over the logits' end (38.25 MB)
])
def test_argmax_argument_checks(over, status):
    assert call_argmax(argmax_args(**over)) == status
    assert da.qknorm_rope_attn_last_hip_error() == 0


def test_argmax_empty_batch_is_noop():
    assert call_argmax(argmax_args(num_rows=0, logits=None, out_index=None, workspace=None)) == da.QKRA_OK


def mixed_args(**over):
    """A prefill half at BASE and a decode half 1 GiB above it (fake device addresses: only the host checks run)."""
    cfg = over.pop("cfg", da.make_config(32, 8, 128, da.QKRA_BF16))
    g = 1024 * MB
    a = dict(q_norm_weight=BASE + 64 * MB, k_norm_weight=BASE + 65 * MB,
             p_qkv=BASE, p_positions=BASE + 66 * MB, cu_seqlens=BASE + 67 * MB, num_tokens=64, num_prefill_seqs=1,
             max_seqlen=64, p_k=BASE + 100 * MB, p_v=BASE + 200 * MB, p_cap=64, p_out=BASE + 300 * MB,
             p_ws=BASE + 400 * MB, p_ws_bytes=1 << 20,
             d_qkv=BASE + g, d_positions=BASE + g + 66 * MB, cache_lens=BASE + g + 67 * MB, num_decode_seqs=4,
             max_cache_len=100, d_k=BASE + g + 100 * MB, d_v=BASE + g + 200 * MB, d_cap=101, d_out=BASE + g + 300 * MB,
             d_ws=BASE + g + 400 * MB, d_ws_bytes=16 * MB, stream=0)
    a.update(over)
    return cfg, a


def call_mixed(cfg, a):
    return da.qknorm_rope_attn_mixed_step(
        cfg, a["q_norm_weight"], a["k_norm_weight"], a["p_qkv"], a["p_positions"], a["cu_seqlens"], a["num_tokens"],
        a["num_prefill_seqs"], a["max_seqlen"], a["p_k"], a["p_v"], a["p_cap"], a["p_out"], a["p_ws"],
        a["p_ws_bytes"], a["d_qkv"], a["d_positions"], a["cache_lens"], a["num_decode_seqs"], a["max_cache_len"],
        a["d_k"], a["d_v"], a["d_cap"], a["d_out"], a["d_ws"], a["d_ws_bytes"], a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(d_cap=100), da.QKRA_ERR_CAPACITY),                                   # decode half: no room for the token
    (dict(d_ws_bytes=1024), da.QKRA_ERR_WORKSPACE_TOO_SMALL),
    (dict(max_seqlen=65), da.QKRA_ERR_INVALID_ARGUMENT),                       # prefill half
    (dict(p_cap=63), da.QKRA_ERR_CAPACITY),
    (dict(num_tokens=-1), da.QKRA_ERR_INVALID_ARGUMENT),
    (dict(d_out=BASE + 300 * MB), da.QKRA_ERR_ALIASING),                       # both outputs in one buffer
    (dict(d_k=BASE + 100 * MB + 4096), da.QKRA_ERR_ALIASING),                  # decode cache over the prefill cache
    (dict(p_ws=BASE + 1024 * MB), da.QKRA_ERR_ALIASING),                       # prefill workspace over decode qkv
    (dict(d_ws=BASE + 4096), da.QKRA_ERR_ALIASING),                            # decode workspace over prefill qkv
])
def test_mixed_step_argument_checks(over, status):
    cfg, a = mixed_args(**over)
    assert call_mixed(cfg, a) == status
    assert da.qknorm_rope_attn_last_hip_error() == 0  # rejected before any launch


def test_mixed_step_with_both_halves_empty_is_noop():
    cfg, a = mixed_args(num_tokens=0, num_decode_seqs=0)
    assert call_mixed(cfg, a) == da.QKRA_OK
    assert da.qknorm_rope_attn_kernel_name(11) == "fused_step_attn"


@pytest.mark.skipif(torch.cuda.is_available(), reason="the fake addresses would reach a kernel launch on a GPU")
def test_mixed_step_workspaces_from_one_arena():
    """Both workspaces carved from one arena, each declared as the rest of it: the declared ranges overlap, the
    bytes each half uses do not, so the checks pass as they do for prefill then decode (here the launch itself
    then fails, as there is no GPU)."""
    cfg, a = mixed_args()
    p_need = da.qknorm_rope_attn_workspace_bytes(cfg, da.QKRA_MODE_PREFILL, a["num_tokens"], a["max_seqlen"])
    arena, arena_bytes = BASE + 400 * MB, 64 * MB
    a.update(p_ws=arena, p_ws_bytes=arena_bytes, d_ws=arena + p_need, d_ws_bytes=arena_bytes - p_need)
    status = on_own_thread(lambda: call_mixed(cfg, a))
    assert status != da.QKRA_ERR_ALIASING
    assert status in (da.QKRA_OK, da.QKRA_ERR_HIP)
    # The decode workspace starting inside the bytes the prefill half uses is still refused.
    a.update(d_ws=arena + p_need - 256)
    assert call_mixed(cfg, a) == da.QKRA_ERR_ALIASING


def test_decode_noalloc_refuses_sizes_past_its_scratch():
    """The no-allocation decode takes its workspace from a fixed array; a call that needs more is refused with its
    own status before anything touches the GPU (so this runs without one)."""
    cfg = da.make_config(32, 8, 128, da.QKRA_BF16)
    need = da.qknorm_rope_attn_workspace_bytes(cfg, da.QKRA_MODE_DECODE, 4096, 100)
    assert need > da.QKRA_NOALLOC_SCRATCH_BYTES
    st = da.qknorm_rope_attn_decode_noalloc(cfg, BASE, BASE + 64 * MB, BASE + 65 * MB, BASE + 66 * MB, BASE + 67 * MB,
                                            4096, 100, BASE + 100 * MB, BASE + 200 * MB, 101, BASE + 300 * MB, 0)
    assert st == da.QKRA_ERR_SCRATCH_LIMIT
    assert "scratch" in da.qknorm_rope_attn_status_string(st)
    # fp32 partials grow with the longest cache: a handful of long requests is already too much.
    cfg32 = da.make_config(32, 8, 128, da.QKRA_FP32)
    assert da.qknorm_rope_attn_workspace_bytes(cfg32, da.QKRA_MODE_DECODE, 64, 65536) > da.QKRA_NOALLOC_SCRATCH_BYTES
    st = da.qknorm_rope_attn_decode_noalloc(cfg32, BASE, BASE + 64 * MB, BASE + 65 * MB, BASE + 66 * MB,
                                            BASE + 67 * MB, 64, 65536, BASE + 100 * MB, BASE + 200 * MB, 65537,
                                            BASE + 300 * MB, 0)
    assert st == da.QKRA_ERR_SCRATCH_LIMIT
    # An empty batch is a no-op; bad arguments keep their own status.
    assert da.qknorm_rope_attn_decode_noalloc(cfg, None, None, None, None, None, 0, 0, None, None, 1, None, 0) == 0
    assert da.qknorm_rope_attn_decode_noalloc(cfg, BASE, BASE, BASE, BASE, BASE, -1, 0, BASE, BASE, 1, BASE, 0) == \
        da.QKRA_ERR_INVALID_ARGUMENT


# ---- paged caches -------------------------------------------------------------------

def paged_decode_args(**over):
    """Four decodes on a paged pool of 40 pages of 64 slots (fake device addresses: host checks only)."""
    cfg = over.pop("cfg", da.make_config(32, 8, 128, da.QKRA_BF16))
    cache = dict(k_pool=BASE + 100 * MB, v_pool=BASE + 200 * MB, block_table=BASE + 68 * MB, num_pages=40,
                 page_size=64, pages_per_seq=10)
    for k in list(over):
        if k in cache:
            cache[k] = over.pop(k)
    a = dict(qkv=BASE, q_norm_weight=BASE + 64 * MB, k_norm_weight=BASE + 65 * MB, positions=BASE + 66 * MB,
             cache_lens=BASE + 67 * MB, num_seqs=4, max_cache_len=639, out=BASE + 300 * MB, workspace=BASE + 400 * MB,
             workspace_bytes=64 * MB, stream=0)
    a.update(over)
    return cfg, da.make_paged_cache(**cache), a


def call_paged_decode(cfg, cache, a):
    return da.qknorm_rope_attn_decode_paged(cfg, a["qkv"], a["q_norm_weight"], a["k_norm_weight"], a["positions"],
                                            a["cache_lens"], a["num_seqs"], a["max_cache_len"], cache, a["out"],
                                            a["workspace"], a["workspace_bytes"], a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(page_size=32), da.QKRA_ERR_UNSUPPORTED),                 # pages must hold 64..1024 slots
    (dict(page_size=96), da.QKRA_ERR_UNSUPPORTED),                 # and a power of two
    (dict(page_size=2048), da.QKRA_ERR_UNSUPPORTED),
    (dict(num_pages=0), da.QKRA_ERR_INVALID_ARGUMENT),
    (dict(pages_per_seq=0), da.QKRA_ERR_INVALID_ARGUMENT),
    (dict(block_table=None), da.QKRA_ERR_INVALID_ARGUMENT),
    (dict(block_table=BASE + 68 * MB + 2), da.QKRA_ERR_INVALID_ARGUMENT),   # misaligned table
    (dict(max_cache_len=640), da.QKRA_ERR_CAPACITY),               # 10 pages of 64 hold 640 slots: no room
    (dict(out=BASE + 68 * MB), da.QKRA_ERR_ALIASING),              # out over the block table
    (dict(workspace=BASE + 100 * MB + 4096), da.QKRA_ERR_ALIASING),  # workspace inside the K pool
    (dict(v_pool=BASE + 100 * MB + 64), da.QKRA_ERR_ALIASING),     # pools overlap
])
def test_paged_decode_argument_checks(over, status):
    cfg, cache, a = paged_decode_args(**over)
    assert call_paged_decode(cfg, cache, a) == status
    assert da.qknorm_rope_attn_last_hip_error() == 0


def test_paged_calls_need_a_descriptor_and_accept_empty_batches():
    cfg, cache, a = paged_decode_args()
    assert da.qknorm_rope_attn_decode_paged(cfg, a["qkv"], a["q_norm_weight"], a["k_norm_weight"], a["positions"],
                                            a["cache_lens"], 4, 100, None, a["out"], a["workspace"],
                                            a["workspace_bytes"], 0) == da.QKRA_ERR_INVALID_ARGUMENT
    assert da.qknorm_rope_attn_decode_paged(cfg, None, None, None, None, None, 0, 0, None, None, None, 0, 0) == 0
    bad = da.make_paged_cache(BASE, BASE, BASE, 1, 64, 1)
    bad.reserved = 1
    assert call_paged_decode(cfg, bad, a) == da.QKRA_ERR_INVALID_ARGUMENT
    # The append: capacity counts the history plus the chunk; a null cache_lens (a prefill) needs max_cache_len 0.
    f = da.qknorm_rope_attn_prefill_append_paged
    args = (cfg, BASE, BASE + 64 * MB, BASE + 65 * MB, BASE + 66 * MB, BASE + 69 * MB)
    assert f(*args, BASE + 67 * MB, 64, 1, 64, 577, cache, BASE + 300 * MB, BASE + 400 * MB, 64 * MB, 0) == \
        da.QKRA_ERR_CAPACITY
    assert f(*args, None, 64, 1, 64, 5, cache, BASE + 300 * MB, BASE + 400 * MB, 64 * MB, 0) == \
        da.QKRA_ERR_INVALID_ARGUMENT
    assert f(*args, None, 0, 0, 0, 0, None, None, None, 0, 0) == 0
    assert da.qknorm_rope_attn_last_hip_error() == 0


def test_weight_bound_field_and_unshifted_limit():
    # The limit: 48 / (1.02 * D * log2(e) / sqrt(D)) -- 2.88 for D = 128, 4.08 for D = 64.
    assert da.qknorm_rope_attn_unshifted_weight_limit(128) == pytest.approx(48 / (1.02 * 128 * 1.4426950408889634
                                                                                  / 128 ** 0.5), rel=1e-6)
    assert da.qknorm_rope_attn_unshifted_weight_limit(64) == pytest.approx(4.0797, rel=1e-3)
    assert da.qknorm_rope_attn_unshifted_weight_limit(96) == 0.0
    for bad in (-1.0, float("nan"), float("inf")):
        cfg, a = prefill_args(cfg=da.make_config(32, 8, 128, da.QKRA_BF16, qk_weight_bound=bad))
        assert call_prefill(cfg, a) == da.QKRA_ERR_INVALID_ARGUMENT
