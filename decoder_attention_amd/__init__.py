"""QK-RMSNorm + RoPE + causal grouped-query attention for MI355X (gfx950).

The computation lives in the HIP library ``libqknorm_rope_attn.so`` (C ABI in
``include/qknorm_rope_attn.h``); this package binds it and adds conveniences
that allocate outputs and workspace with PyTorch before calling it.  PyTorch supplies device memory and the current stream only.
"""

from __future__ import annotations

from .binding import (  # noqa: F401
    QKRA_BF16,
    QKRA_FP32,
    QKRA_OK,
    QKRA_ERR_INVALID_ARGUMENT,
    QKRA_ERR_UNSUPPORTED,
    QKRA_ERR_CAPACITY,
    QKRA_ERR_WORKSPACE_TOO_SMALL,
    QKRA_ERR_ALIASING,
    QKRA_ERR_HIP,
    QKRA_ERR_SCRATCH_LIMIT,
    QKRA_NOALLOC_SCRATCH_BYTES,
    QKRA_MODE_PREFILL,
    QKRA_MODE_DECODE,
    QkraConfig,
    QkraError,
    QkraPagedCache,
    make_paged_cache,
    check,
    exported_symbols,
    calibration_lib,
    calibration_symbols,
    qkra_calibrate_stream_read,
    qkra_calibrate_stream_copy,
    qkra_calibrate_mfma_bf16,
    qkra_calibrate_mfma_flop,
    phase_stamps_symbols,
    qkra_phase_stamps_bytes,
    qkra_phase_stamps_clear,
    qkra_phase_stamps_read,
    select_library,
    lib,
    make_config,
    qknorm_rope_attn_prefill,
    qknorm_rope_attn_prefill_append,
    qknorm_rope_attn_decode,
    qknorm_rope_attn_decode_noalloc,
    qknorm_rope_attn_decode_paged,
    qknorm_rope_attn_prefill_append_paged,
    qknorm_rope_attn_mixed_step,
    qknorm_rope_attn_workspace_bytes,
    qknorm_rope_attn_status_string,
    qknorm_rope_attn_last_hip_error,
    qknorm_rope_attn_unshifted_weight_limit,
    qknorm_rope_attn_version,
    qknorm_rope_attn_set_kernel_timing,
    qknorm_rope_attn_read_kernel_timing,
    qknorm_rope_attn_kernel_name,
    qknorm_rope_attn_fused_add_rmsnorm,
    qknorm_rope_attn_gather_last,
    qknorm_rope_attn_argmax_workspace_bytes,
    qknorm_rope_attn_argmax,
)


def _require_device(*tensors):
    for t in tensors:
        if not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")


def prefill(cfg: QkraConfig, qkv, q_norm_weight, k_norm_weight, positions, cu_seqlens, max_seqlen: int,
            k_cache, v_cache, out=None, workspace=None, stream=None):
    """Runs ``qknorm_rope_attn_prefill``; returns (out [N, Hq*D], workspace)."""
    import torch

    _require_device(qkv, q_norm_weight, k_norm_weight, positions, cu_seqlens, k_cache, v_cache)
    n = qkv.shape[0]
    b = cu_seqlens.shape[0] - 1
    if out is None:
        out = torch.empty((n, cfg.num_q_heads * cfg.head_dim), dtype=qkv.dtype, device=qkv.device)
    need = qknorm_rope_attn_workspace_bytes(cfg, QKRA_MODE_PREFILL, n, max_seqlen)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=qkv.device)
    status = qknorm_rope_attn_prefill(cfg, qkv, q_norm_weight, k_norm_weight, positions, cu_seqlens, n, b,
                                      max_seqlen, k_cache, v_cache, k_cache.shape[2], out, workspace,
                                      workspace.numel() * workspace.element_size(), stream)
    check(status, "qknorm_rope_attn_prefill")
    return out, workspace


def prefill_append(cfg: QkraConfig, qkv, q_norm_weight, k_norm_weight, positions, cu_seqlens, cache_lens,
                   max_seqlen: int, max_cache_len: int, k_cache, v_cache, out=None, workspace=None, stream=None):
    """Runs ``qknorm_rope_attn_prefill_append``; returns (out [N, Hq*D], workspace)."""
    import torch

    _require_device(qkv, q_norm_weight, k_norm_weight, positions, cu_seqlens, cache_lens, k_cache, v_cache)
    n = qkv.shape[0]
    b = cu_seqlens.shape[0] - 1
    if out is None:
        out = torch.empty((n, cfg.num_q_heads * cfg.head_dim), dtype=qkv.dtype, device=qkv.device)
    need = qknorm_rope_attn_workspace_bytes(cfg, QKRA_MODE_PREFILL, n, max_seqlen)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=qkv.device)
    status = qknorm_rope_attn_prefill_append(cfg, qkv, q_norm_weight, k_norm_weight, positions, cu_seqlens,
                                             cache_lens, n, b, max_seqlen, max_cache_len, k_cache, v_cache,
                                             k_cache.shape[2], out, workspace,
                                             workspace.numel() * workspace.element_size(), stream)
    check(status, "qknorm_rope_attn_prefill_append")
    return out, workspace


def decode(cfg: QkraConfig, qkv, q_norm_weight, k_norm_weight, positions, cache_lens, max_cache_len: int,
           k_cache, v_cache, out=None, workspace=None, stream=None):
    """Runs ``qknorm_rope_attn_decode``; returns (out [B, Hq*D], workspace)."""
    import torch

    _require_device(qkv, q_norm_weight, k_norm_weight, positions, cache_lens, k_cache, v_cache)
    b = qkv.shape[0]
    if out is None:
        out = torch.empty((b, cfg.num_q_heads * cfg.head_dim), dtype=qkv.dtype, device=qkv.device)
    need = qknorm_rope_attn_workspace_bytes(cfg, QKRA_MODE_DECODE, b, max_cache_len)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=qkv.device)
    status = qknorm_rope_attn_decode(cfg, qkv, q_norm_weight, k_norm_weight, positions, cache_lens, b,
                                     max_cache_len, k_cache, v_cache, k_cache.shape[2], out, workspace,
                                     workspace.numel() * workspace.element_size(), stream)
    check(status, "qknorm_rope_attn_decode")
    return out, workspace


def decode_noalloc(cfg: QkraConfig, qkv, q_norm_weight, k_norm_weight, positions, cache_lens, max_cache_len: int,
                   k_cache, v_cache, out, stream=None):
    """Runs ``qknorm_rope_attn_decode_noalloc`` into the caller's ``out`` (the library's fixed scratch serves as
    the workspace; nothing is allocated); returns out."""
    _require_device(qkv, q_norm_weight, k_norm_weight, positions, cache_lens, k_cache, v_cache, out)
    status = qknorm_rope_attn_decode_noalloc(cfg, qkv, q_norm_weight, k_norm_weight, positions, cache_lens,
                                             qkv.shape[0], max_cache_len, k_cache, v_cache, k_cache.shape[2], out,
                                             stream)
    check(status, "qknorm_rope_attn_decode_noalloc")
    return out


def decode_paged(cfg: QkraConfig, qkv, q_norm_weight, k_norm_weight, positions, cache_lens, max_cache_len: int,
                 k_pool, v_pool, block_table, page_size: int, out=None, workspace=None, stream=None):
    """Runs ``qknorm_rope_attn_decode_paged`` (pools [num_pages, Hkv, page_size, D], block_table int32
    [B, pages_per_seq]); returns (out [B, Hq*D], workspace)."""
    import torch

    _require_device(qkv, q_norm_weight, k_norm_weight, positions, cache_lens, k_pool, v_pool, block_table)
    b = qkv.shape[0]
    if out is None:
        out = torch.empty((b, cfg.num_q_heads * cfg.head_dim), dtype=qkv.dtype, device=qkv.device)
    need = qknorm_rope_attn_workspace_bytes(cfg, QKRA_MODE_DECODE, b, max_cache_len)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=qkv.device)
    cache = make_paged_cache(k_pool, v_pool, block_table, k_pool.shape[0], page_size, block_table.shape[1])
    status = qknorm_rope_attn_decode_paged(cfg, qkv, q_norm_weight, k_norm_weight, positions, cache_lens, b,
                                           max_cache_len, cache, out, workspace,
                                           workspace.numel() * workspace.element_size(), stream)
    check(status, "qknorm_rope_attn_decode_paged")
    return out, workspace


def prefill_append_paged(cfg: QkraConfig, qkv, q_norm_weight, k_norm_weight, positions, cu_seqlens, cache_lens,
                         max_seqlen: int, max_cache_len: int, k_pool, v_pool, block_table, page_size: int, out=None,
                         workspace=None, stream=None):
    """Runs ``qknorm_rope_attn_prefill_append_paged`` (cache_lens None: a prefill into the paged cache); returns
    (out [N, Hq*D], workspace)."""
    import torch

    _require_device(qkv, q_norm_weight, k_norm_weight, positions, cu_seqlens, k_pool, v_pool, block_table)
    if cache_lens is not None:
        _require_device(cache_lens)
    n = qkv.shape[0]
    b = cu_seqlens.shape[0] - 1
    if out is None:
        out = torch.empty((n, cfg.num_q_heads * cfg.head_dim), dtype=qkv.dtype, device=qkv.device)
    need = qknorm_rope_attn_workspace_bytes(cfg, QKRA_MODE_PREFILL, n, max_seqlen)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=qkv.device)
    cache = make_paged_cache(k_pool, v_pool, block_table, k_pool.shape[0], page_size, block_table.shape[1])
    status = qknorm_rope_attn_prefill_append_paged(cfg, qkv, q_norm_weight, k_norm_weight, positions, cu_seqlens,
                                                   cache_lens, n, b, max_seqlen, max_cache_len, cache, out,
                                                   workspace, workspace.numel() * workspace.element_size(), stream)
    check(status, "qknorm_rope_attn_prefill_append_paged")
    return out, workspace


def mixed_step(cfg: QkraConfig, q_norm_weight, k_norm_weight, prefill_qkv, prefill_positions, cu_seqlens,
               max_seqlen: int, prefill_k_cache, prefill_v_cache, decode_qkv, decode_positions, cache_lens,
               max_cache_len: int, decode_k_cache, decode_v_cache, prefill_out=None, prefill_workspace=None,
               decode_out=None, decode_workspace=None, stream=None):
    """Runs ``qknorm_rope_attn_mixed_step``; returns (prefill out, decode out, prefill workspace, decode workspace)."""
    import torch

    _require_device(prefill_qkv, q_norm_weight, k_norm_weight, prefill_positions, cu_seqlens, prefill_k_cache,
                    prefill_v_cache, decode_qkv, decode_positions, cache_lens, decode_k_cache, decode_v_cache)
    n, b = prefill_qkv.shape[0], decode_qkv.shape[0]
    width = cfg.num_q_heads * cfg.head_dim
    if prefill_out is None:
        prefill_out = torch.empty((n, width), dtype=prefill_qkv.dtype, device=prefill_qkv.device)
    if decode_out is None:
        decode_out = torch.empty((b, width), dtype=decode_qkv.dtype, device=decode_qkv.device)
    if prefill_workspace is None:
        need = qknorm_rope_attn_workspace_bytes(cfg, QKRA_MODE_PREFILL, n, max_seqlen)
        prefill_workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=prefill_qkv.device)
    if decode_workspace is None:
        need = qknorm_rope_attn_workspace_bytes(cfg, QKRA_MODE_DECODE, b, max_cache_len)
        decode_workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=decode_qkv.device)
    status = qknorm_rope_attn_mixed_step(
        cfg, q_norm_weight, k_norm_weight, prefill_qkv, prefill_positions, cu_seqlens, n, cu_seqlens.shape[0] - 1,
        max_seqlen, prefill_k_cache, prefill_v_cache, prefill_k_cache.shape[2], prefill_out, prefill_workspace,
        prefill_workspace.numel() * prefill_workspace.element_size(), decode_qkv, decode_positions, cache_lens, b,
        max_cache_len, decode_k_cache, decode_v_cache, decode_k_cache.shape[2], decode_out, decode_workspace,
        decode_workspace.numel() * decode_workspace.element_size(), stream)
    check(status, "qknorm_rope_attn_mixed_step")
    return prefill_out, decode_out, prefill_workspace, decode_workspace


def _dtype_code(t):
    import torch

    if t.dtype == torch.bfloat16:
        return QKRA_BF16
    if t.dtype == torch.float32:
        return QKRA_FP32
    raise ValueError(f"unsupported dtype {t.dtype}")


def fused_add_rmsnorm(x, residual, weight, eps: float, has_residual: bool, out=None, stream=None):
    """Runs ``qknorm_rope_attn_fused_add_rmsnorm``; returns out [N, C] (residual is updated in place)."""
    import torch

    _require_device(x, residual, weight)
    if out is None:
        out = torch.empty_like(x)
    status = qknorm_rope_attn_fused_add_rmsnorm(_dtype_code(x), eps, x, residual, has_residual, weight, out,
                                                x.shape[0], x.shape[1], stream)
    check(status, "qknorm_rope_attn_fused_add_rmsnorm")
    return out


def gather_last(hidden, cu_seqlens, out=None, stream=None):
    """Runs ``qknorm_rope_attn_gather_last``; returns [B, C] (rows of empty requests are left as allocated)."""
    import torch

    _require_device(hidden, cu_seqlens)
    b = cu_seqlens.shape[0] - 1
    if out is None:
        out = torch.zeros((b, hidden.shape[1]), dtype=hidden.dtype, device=hidden.device)
    status = qknorm_rope_attn_gather_last(_dtype_code(hidden), hidden, cu_seqlens, hidden.shape[0], b,
                                          hidden.shape[1], out, stream)
    check(status, "qknorm_rope_attn_gather_last")
    return out


def argmax(logits, out=None, workspace=None, stream=None):
    """Runs ``qknorm_rope_attn_argmax`` on a [B, V] tensor (rows may be strided); returns int32 [B]."""
    import torch

    if not logits.is_cuda or logits.stride(1) != 1:
        raise ValueError("logits must be a GPU tensor with contiguous rows")
    b, v = logits.shape
    if out is None:
        out = torch.empty((b,), dtype=torch.int32, device=logits.device)
    need = qknorm_rope_attn_argmax_workspace_bytes(b, v)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=logits.device)
    status = qknorm_rope_attn_argmax(_dtype_code(logits), logits, b, v, logits.stride(0), out, workspace,
                                     workspace.numel(), stream)
    check(status, "qknorm_rope_attn_argmax")
    return out
