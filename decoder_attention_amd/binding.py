"""ctypes binding of the C ABI declared in ``include/qknorm_rope_attn.h``.

Argument marshalling only: tensors become device pointers, the stream becomes
a ``hipStream_t``.  Every step of the computation runs in the HIP library; if
the library is not built, loading it raises instead of falling back to
anything else.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

from .build import LIB_PATH

QKRA_BF16 = 0
QKRA_FP32 = 1

QKRA_OK = 0
QKRA_ERR_INVALID_ARGUMENT = 1
QKRA_ERR_UNSUPPORTED = 2
QKRA_ERR_CAPACITY = 3
QKRA_ERR_WORKSPACE_TOO_SMALL = 4
QKRA_ERR_ALIASING = 5
QKRA_ERR_HIP = 6
QKRA_ERR_SCRATCH_LIMIT = 7

QKRA_NOALLOC_SCRATCH_BYTES = 16 << 20

QKRA_MODE_PREFILL = 0
QKRA_MODE_DECODE = 1


class QkraConfig(ctypes.Structure):
    _fields_ = [
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("rms_eps", ctypes.c_float),
        ("qk_weight_bound", ctypes.c_float),
        ("rope_base", ctypes.c_double),
    ]


class QkraPagedCache(ctypes.Structure):
    _fields_ = [
        ("k_pool", ctypes.c_void_p),
        ("v_pool", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
        ("num_pages", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("pages_per_seq", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


class QkraError(RuntimeError):
    def __init__(self, status: int, where: str = ""):
        self.status = status
        msg = f"{where}: " if where else ""
        msg += f"status {status} ({qknorm_rope_attn_status_string(status)})"
        if status == QKRA_ERR_HIP:
            msg += f", hipError {qknorm_rope_attn_last_hip_error()}"
        super().__init__(msg)


_lib: Optional[ctypes.CDLL] = None

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_SZ = ctypes.c_size_t

_SIGNATURES = {
    "qknorm_rope_attn_prefill": (_I32, [ctypes.POINTER(QkraConfig), _P, _P, _P, _P, _P, _I32, _I32, _I32, _P, _P,
                                        _I32, _P, _P, _SZ, _P]),
    "qknorm_rope_attn_prefill_append": (_I32, [ctypes.POINTER(QkraConfig), _P, _P, _P, _P, _P, _P, _I32, _I32, _I32,
                                               _I32, _P, _P, _I32, _P, _P, _SZ, _P]),
    "qknorm_rope_attn_decode": (_I32, [ctypes.POINTER(QkraConfig), _P, _P, _P, _P, _P, _I32, _I32, _P, _P, _I32,
                                       _P, _P, _SZ, _P]),
    "qknorm_rope_attn_decode_noalloc": (_I32, [ctypes.POINTER(QkraConfig), _P, _P, _P, _P, _P, _I32, _I32, _P, _P,
                                               _I32, _P, _P]),
    "qknorm_rope_attn_decode_paged": (_I32, [ctypes.POINTER(QkraConfig), _P, _P, _P, _P, _P, _I32, _I32,
                                             ctypes.POINTER(QkraPagedCache), _P, _P, _SZ, _P]),
    "qknorm_rope_attn_prefill_append_paged": (_I32, [ctypes.POINTER(QkraConfig), _P, _P, _P, _P, _P, _P, _I32, _I32,
                                                     _I32, _I32, ctypes.POINTER(QkraPagedCache), _P, _P, _SZ, _P]),
    "qknorm_rope_attn_mixed_step": (_I32, [ctypes.POINTER(QkraConfig), _P, _P, _P, _P, _P, _I32, _I32, _I32, _P, _P,
                                           _I32, _P, _P, _SZ, _P, _P, _P, _I32, _I32, _P, _P, _I32, _P, _P, _SZ, _P]),
    "qknorm_rope_attn_workspace_bytes": (_SZ, [ctypes.POINTER(QkraConfig), _I32, _I32, _I32]),
    "qknorm_rope_attn_status_string": (ctypes.c_char_p, [_I32]),
    "qknorm_rope_attn_last_hip_error": (_I32, []),
    "qknorm_rope_attn_unshifted_weight_limit": (ctypes.c_float, [_I32]),
    "qknorm_rope_attn_version": (_I32, []),
    "qknorm_rope_attn_set_kernel_timing": (_I32, [_I32]),
    "qknorm_rope_attn_read_kernel_timing": (_I32, [ctypes.POINTER(ctypes.c_double),
                                                   ctypes.POINTER(ctypes.c_int64), _I32]),
    "qknorm_rope_attn_kernel_name": (ctypes.c_char_p, [_I32]),
    "qknorm_rope_attn_fused_add_rmsnorm": (_I32, [_I32, ctypes.c_float, _P, _P, _I32, _P, _P, _I32, _I32, _P]),
    "qknorm_rope_attn_gather_last": (_I32, [_I32, _P, _P, _I32, _I32, _I32, _P, _P]),
    "qknorm_rope_attn_argmax_workspace_bytes": (_SZ, [_I32, _I32]),
    "qknorm_rope_attn_argmax": (_I32, [_I32, _P, _I32, _I32, ctypes.c_int64, _P, _P, _SZ, _P]),
}


_lib_path = LIB_PATH


def select_library(path: str) -> None:
    """Load `path`, another build of the same sources (the phase-stamps profiling build), in place of the
    normal library.  Must come before the first call into the library."""
    global _lib_path
    if _lib is not None and os.path.abspath(path) != os.path.abspath(_lib_path):
        raise RuntimeError(f"{_lib_path} is already loaded")
    _lib_path = path


def lib() -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_lib_path):
            raise RuntimeError(
                f"HIP library {_lib_path} is missing; build it first "
                "(python -c 'import __graft_entry__ as g; g.build()' or python decoder_attention_amd/build.py)")
        handle = ctypes.CDLL(_lib_path)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def exported_symbols():
    return sorted(_SIGNATURES)


# ---- the roofline calibration library (include/qkra_calibrate.h) ---------------
_calib = None
_CALIB_SIGNATURES = {
    "qkra_calibrate_stream_read": (_I32, [_P, _SZ, _P, _I32, _P]),
    "qkra_calibrate_stream_copy": (_I32, [_P, _P, _SZ, _P]),
    "qkra_calibrate_mfma_bf16": (_I32, [ctypes.c_int64, _P, _I32, _P]),
    "qkra_calibrate_mfma_flop": (_SZ, [ctypes.c_int64, _I32]),
}


def calibration_lib() -> ctypes.CDLL:
    """Load libqkra_calibrate.so (raises if it has not been built)."""
    global _calib
    if _calib is None:
        from .build import CALIB_LIB_PATH

        if not os.path.exists(CALIB_LIB_PATH):
            raise RuntimeError(f"calibration library {CALIB_LIB_PATH} is missing; build it first")
        handle = ctypes.CDLL(CALIB_LIB_PATH)
        for name, (res, args) in _CALIB_SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _calib = handle
    return _calib


def calibration_symbols():
    return sorted(_CALIB_SIGNATURES)


def qkra_calibrate_stream_read(buf, nbytes: int, sink, workgroups: int, stream=None) -> int:
    return calibration_lib().qkra_calibrate_stream_read(_ptr(buf), int(nbytes), _ptr(sink), int(workgroups),
                                                        _stream(stream))


def qkra_calibrate_stream_copy(src, dst, nbytes: int, stream=None) -> int:
    return calibration_lib().qkra_calibrate_stream_copy(_ptr(src), _ptr(dst), int(nbytes), _stream(stream))


def qkra_calibrate_mfma_bf16(iterations: int, sink, workgroups: int, stream=None) -> int:
    return calibration_lib().qkra_calibrate_mfma_bf16(int(iterations), _ptr(sink), int(workgroups), _stream(stream))


def qkra_calibrate_mfma_flop(iterations: int, workgroups: int) -> int:
    return int(calibration_lib().qkra_calibrate_mfma_flop(int(iterations), int(workgroups)))


# ---- the profiling build's phase stamps (include/qkra_phase_stamps.h) ----------
_STAMPS_SIGNATURES = {
    "qkra_phase_stamps_read": (_I32, [_P, _SZ]),
    "qkra_phase_stamps_clear": (_I32, [_P]),
    "qkra_phase_stamps_bytes": (_SZ, []),
}


def phase_stamps_symbols():
    return sorted(_STAMPS_SIGNATURES)


def _stamps():
    handle = lib()
    if not hasattr(handle, "qkra_phase_stamps_read"):
        raise RuntimeError(f"{_lib_path} is not the phase-stamps build; select_library() it first")
    for name, (res, args) in _STAMPS_SIGNATURES.items():
        fn = getattr(handle, name)
        fn.restype = res
        fn.argtypes = args
    return handle


def qkra_phase_stamps_bytes() -> int:
    return int(_stamps().qkra_phase_stamps_bytes())


def qkra_phase_stamps_clear(stream=None) -> int:
    return _stamps().qkra_phase_stamps_clear(_stream(stream))


def qkra_phase_stamps_read(dst, nbytes: int) -> int:
    """`dst`: a host address (int) or a CPU tensor / NumPy array with the buffer protocol's data pointer."""
    ptr = dst if isinstance(dst, int) else (dst.ctypes.data if hasattr(dst, "ctypes") else dst.data_ptr())
    return _stamps().qkra_phase_stamps_read(ptr, int(nbytes))


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_config(num_q_heads: int, num_kv_heads: int, head_dim: int, dtype=QKRA_BF16, rms_eps: float = 1e-6,
                rope_base: float = 1e6, qk_weight_bound: float = 0.0) -> QkraConfig:
    if not isinstance(dtype, int):
        import torch

        dtype = {torch.bfloat16: QKRA_BF16, torch.float32: QKRA_FP32}[dtype]
    return QkraConfig(int(num_q_heads), int(num_kv_heads), int(head_dim), int(dtype), float(rms_eps),
                      float(qk_weight_bound), float(rope_base))


# ---- the C ABI, one Python function per exported symbol -------------------

def qknorm_rope_attn_prefill(cfg: QkraConfig, qkv, q_norm_weight, k_norm_weight, positions, cu_seqlens,
                             num_tokens: int, num_seqs: int, max_seqlen: int, k_cache, v_cache,
                             cache_capacity: int, out, workspace, workspace_bytes: int, stream=None) -> int:
    return lib().qknorm_rope_attn_prefill(
        ctypes.byref(cfg), _ptr(qkv), _ptr(q_norm_weight), _ptr(k_norm_weight), _ptr(positions), _ptr(cu_seqlens),
        int(num_tokens), int(num_seqs), int(max_seqlen), _ptr(k_cache), _ptr(v_cache), int(cache_capacity),
        _ptr(out), _ptr(workspace), int(workspace_bytes), _stream(stream))


def qknorm_rope_attn_prefill_append(cfg: QkraConfig, qkv, q_norm_weight, k_norm_weight, positions, cu_seqlens,
                                    cache_lens, num_tokens: int, num_seqs: int, max_seqlen: int,
                                    max_cache_len: int, k_cache, v_cache, cache_capacity: int, out, workspace,
                                    workspace_bytes: int, stream=None) -> int:
    return lib().qknorm_rope_attn_prefill_append(
        ctypes.byref(cfg), _ptr(qkv), _ptr(q_norm_weight), _ptr(k_norm_weight), _ptr(positions), _ptr(cu_seqlens),
        _ptr(cache_lens), int(num_tokens), int(num_seqs), int(max_seqlen), int(max_cache_len), _ptr(k_cache),
        _ptr(v_cache), int(cache_capacity), _ptr(out), _ptr(workspace), int(workspace_bytes), _stream(stream))


def qknorm_rope_attn_mixed_step(cfg: QkraConfig, q_norm_weight, k_norm_weight, prefill_qkv, prefill_positions,
                                cu_seqlens, num_tokens: int, num_prefill_seqs: int, max_seqlen: int, prefill_k_cache,
                                prefill_v_cache, prefill_cache_capacity: int, prefill_out, prefill_workspace,
                                prefill_workspace_bytes: int, decode_qkv, decode_positions, cache_lens,
                                num_decode_seqs: int, max_cache_len: int, decode_k_cache, decode_v_cache,
                                decode_cache_capacity: int, decode_out, decode_workspace, decode_workspace_bytes: int,
                                stream=None) -> int:
    return lib().qknorm_rope_attn_mixed_step(
        ctypes.byref(cfg), _ptr(q_norm_weight), _ptr(k_norm_weight), _ptr(prefill_qkv), _ptr(prefill_positions),
        _ptr(cu_seqlens), int(num_tokens), int(num_prefill_seqs), int(max_seqlen), _ptr(prefill_k_cache),
        _ptr(prefill_v_cache), int(prefill_cache_capacity), _ptr(prefill_out), _ptr(prefill_workspace),
        int(prefill_workspace_bytes), _ptr(decode_qkv), _ptr(decode_positions), _ptr(cache_lens), int(num_decode_seqs),
        int(max_cache_len), _ptr(decode_k_cache), _ptr(decode_v_cache), int(decode_cache_capacity), _ptr(decode_out),
        _ptr(decode_workspace), int(decode_workspace_bytes), _stream(stream))


def qknorm_rope_attn_decode(cfg: QkraConfig, qkv, q_norm_weight, k_norm_weight, positions, cache_lens,
                            num_seqs: int, max_cache_len: int, k_cache, v_cache, cache_capacity: int, out,
                            workspace, workspace_bytes: int, stream=None) -> int:
    return lib().qknorm_rope_attn_decode(
        ctypes.byref(cfg), _ptr(qkv), _ptr(q_norm_weight), _ptr(k_norm_weight), _ptr(positions), _ptr(cache_lens),
        int(num_seqs), int(max_cache_len), _ptr(k_cache), _ptr(v_cache), int(cache_capacity), _ptr(out),
        _ptr(workspace), int(workspace_bytes), _stream(stream))


def qknorm_rope_attn_decode_noalloc(cfg: QkraConfig, qkv, q_norm_weight, k_norm_weight, positions, cache_lens,
                                    num_seqs: int, max_cache_len: int, k_cache, v_cache, cache_capacity: int, out,
                                    stream=None) -> int:
    return lib().qknorm_rope_attn_decode_noalloc(
        ctypes.byref(cfg), _ptr(qkv), _ptr(q_norm_weight), _ptr(k_norm_weight), _ptr(positions), _ptr(cache_lens),
        int(num_seqs), int(max_cache_len), _ptr(k_cache), _ptr(v_cache), int(cache_capacity), _ptr(out),
        _stream(stream))


def make_paged_cache(k_pool, v_pool, block_table, num_pages: int, page_size: int,
                     pages_per_seq: int) -> QkraPagedCache:
    return QkraPagedCache(_ptr(k_pool), _ptr(v_pool), _ptr(block_table), int(num_pages), int(page_size),
                          int(pages_per_seq), 0)


def qknorm_rope_attn_decode_paged(cfg: QkraConfig, qkv, q_norm_weight, k_norm_weight, positions, cache_lens,
                                  num_seqs: int, max_cache_len: int, cache: Optional[QkraPagedCache], out, workspace,
                                  workspace_bytes: int, stream=None) -> int:
    return lib().qknorm_rope_attn_decode_paged(
        ctypes.byref(cfg), _ptr(qkv), _ptr(q_norm_weight), _ptr(k_norm_weight), _ptr(positions), _ptr(cache_lens),
        int(num_seqs), int(max_cache_len), None if cache is None else ctypes.byref(cache), _ptr(out), _ptr(workspace),
        int(workspace_bytes), _stream(stream))


def qknorm_rope_attn_prefill_append_paged(cfg: QkraConfig, qkv, q_norm_weight, k_norm_weight, positions, cu_seqlens,
                                          cache_lens, num_tokens: int, num_seqs: int, max_seqlen: int,
                                          max_cache_len: int, cache: Optional[QkraPagedCache], out, workspace,
                                          workspace_bytes: int, stream=None) -> int:
    return lib().qknorm_rope_attn_prefill_append_paged(
        ctypes.byref(cfg), _ptr(qkv), _ptr(q_norm_weight), _ptr(k_norm_weight), _ptr(positions), _ptr(cu_seqlens),
        _ptr(cache_lens), int(num_tokens), int(num_seqs), int(max_seqlen), int(max_cache_len),
        None if cache is None else ctypes.byref(cache), _ptr(out), _ptr(workspace), int(workspace_bytes),
        _stream(stream))


def qknorm_rope_attn_workspace_bytes(cfg: QkraConfig, mode: int, n: int, max_len: int) -> int:
    return int(lib().qknorm_rope_attn_workspace_bytes(ctypes.byref(cfg), int(mode), int(n), int(max_len)))


def qknorm_rope_attn_status_string(status: int) -> str:
    return lib().qknorm_rope_attn_status_string(int(status)).decode()


def qknorm_rope_attn_last_hip_error() -> int:
    return int(lib().qknorm_rope_attn_last_hip_error())


def qknorm_rope_attn_unshifted_weight_limit(head_dim: int) -> float:
    return float(lib().qknorm_rope_attn_unshifted_weight_limit(int(head_dim)))


def qknorm_rope_attn_version() -> int:
    return int(lib().qknorm_rope_attn_version())


def qknorm_rope_attn_set_kernel_timing(enable) -> int:
    """enable: True (every kernel), False (off), or an int mask over kernel ids."""
    mask = -1 if enable is True else 0 if enable is False else int(enable)
    return int(lib().qknorm_rope_attn_set_kernel_timing(mask))


def qknorm_rope_attn_kernel_name(kernel_id: int) -> str:
    return lib().qknorm_rope_attn_kernel_name(int(kernel_id)).decode()


def qknorm_rope_attn_fused_add_rmsnorm(dtype: int, rms_eps: float, x, residual, has_residual: bool, weight, out,
                                       num_tokens: int, hidden_size: int, stream=None) -> int:
    return lib().qknorm_rope_attn_fused_add_rmsnorm(int(dtype), float(rms_eps), _ptr(x), _ptr(residual),
                                                    1 if has_residual else 0, _ptr(weight), _ptr(out),
                                                    int(num_tokens), int(hidden_size), _stream(stream))


def qknorm_rope_attn_gather_last(dtype: int, hidden, cu_seqlens, num_tokens: int, num_seqs: int, hidden_size: int,
                                 out, stream=None) -> int:
    return lib().qknorm_rope_attn_gather_last(int(dtype), _ptr(hidden), _ptr(cu_seqlens), int(num_tokens),
                                              int(num_seqs), int(hidden_size), _ptr(out), _stream(stream))


def qknorm_rope_attn_argmax_workspace_bytes(num_rows: int, vocab: int) -> int:
    return int(lib().qknorm_rope_attn_argmax_workspace_bytes(int(num_rows), int(vocab)))


def qknorm_rope_attn_argmax(dtype: int, logits, num_rows: int, vocab: int, row_stride: int, out_index, workspace,
                            workspace_bytes: int, stream=None) -> int:
    return lib().qknorm_rope_attn_argmax(int(dtype), _ptr(logits), int(num_rows), int(vocab), int(row_stride),
                                         _ptr(out_index), _ptr(workspace), int(workspace_bytes), _stream(stream))


def qknorm_rope_attn_read_kernel_timing(max_kernels: int = 16):
    """Returns {kernel name: (total ms, launches)} for kernels launched since the last read."""
    ms = (ctypes.c_double * max_kernels)()
    n = (ctypes.c_int64 * max_kernels)()
    count = lib().qknorm_rope_attn_read_kernel_timing(ms, n, int(max_kernels))
    if count < 0:
        raise QkraError(-count, "read_kernel_timing")
    return {qknorm_rope_attn_kernel_name(k): (ms[k], int(n[k])) for k in range(min(count, max_kernels)) if n[k]}


def check(status: int, where: str = "") -> None:
    if status != QKRA_OK:
        raise QkraError(status, where)
