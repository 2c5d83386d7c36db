"""SeerAttention-R decode-time hot path for MI355X (gfx950).

A thin ctypes binding over ``libseer.so`` (C ABI in ``include/seer.h``).  The
functions below only marshal arguments: they check tensor dtypes, devices
and shapes against the ``seer_dims`` they are given, pass raw device
pointers and torch's current HIP stream, and raise ``SeerError`` on a non-OK
status.  Every step of the path runs in the library's HIP kernels; PyTorch
provides device memory and streams only.  If the library is not built, every
call raises -- there is no fallback.

Call order for one decode step of one layer (pages: chapterpal
"SeerAttention-R: Sparse Attention Adaptation for Long Reasoning", Knowl 5
and Knowl 6):

    seer_kcomp_update -> seer_gate_scores -> seer_select_blocks
        -> seer_sparse_decode     (seer_dense_decode is the full baseline)

``DecodeStep`` bundles the buffers and the four calls.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

__all__ = [
    "SeerError", "SeerDims", "lib", "LIB_PATH", "EXPORTED_SYMBOLS",
    "SELECT_TOPK", "SELECT_THRESHOLD", "SELECT_TOPP", "make_dims",
    "seer_kcomp_update", "seer_gate_workspace_bytes", "seer_gate_scores",
    "seer_select_blocks", "seer_decode_workspace_bytes", "seer_workspace_bytes",
    "seer_decode_num_split",
    "seer_sparse_decode", "seer_dense_decode", "seer_sparse_decode_paged",
    "seer_dense_decode_paged", "seer_prefill_workspace_bytes", "seer_prefill_attention",
    "seer_decode_step_workspace_bytes",
    "seer_decode_step", "seer_decode_step_noalloc", "NOALLOC_SCRATCH_BYTES", "SPLIT_BALANCED",
    "seer_status_string", "seer_last_error_message", "seer_version",
    "DecodeStep",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libseer.so")

SEER_OK = 0
SELECT_TOPK = 1
SELECT_THRESHOLD = 2
SELECT_TOPP = 3  # threshold carries the mass p
NOALLOC_SCRATCH_BYTES = 16 << 20  # seer_decode_step_noalloc's static workspace per GPU
SPLIT_BALANCED = -1  # num_split: the fused step's division of uneven selections

EXPORTED_SYMBOLS = (
    "seer_kcomp_update", "seer_gate_workspace_bytes", "seer_gate_scores",
    "seer_select_blocks", "seer_decode_workspace_bytes", "seer_workspace_bytes",
    "seer_decode_num_split",
    "seer_sparse_decode", "seer_dense_decode", "seer_sparse_decode_paged",
    "seer_dense_decode_paged", "seer_prefill_workspace_bytes", "seer_prefill_attention",
    "seer_decode_step_workspace_bytes",
    "seer_decode_step", "seer_decode_step_noalloc", "seer_status_string",
    "seer_last_error_message", "seer_version",
)


class SeerError(RuntimeError):
    def __init__(self, code: int, where: str, detail: str):
        super().__init__(f"{where}: {seer_status_string(code)} ({detail})")
        self.code = code


class SeerDims(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("d_gate", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("max_seq_len", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("kv_stride_b", ctypes.c_int64),
        ("kv_stride_h", ctypes.c_int64),
        ("kv_stride_t", ctypes.c_int64),
    ]

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def nb_max(self) -> int:
        return -(-self.max_seq_len // self.block_size)


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_SIGS = {
    "seer_kcomp_update": (_I32, [ctypes.POINTER(SeerDims), _P, _P, _P, _P, _P, _I32, ctypes.c_double, _P]),
    "seer_gate_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(SeerDims)]),
    "seer_gate_scores": (_I32, [ctypes.POINTER(SeerDims), _P, _P, _P, _P, _P, ctypes.c_double, _P,
                                ctypes.c_size_t, _P, _P]),
    "seer_select_blocks": (_I32, [ctypes.POINTER(SeerDims), _P, _P, _P, _I32, _I32, ctypes.c_float,
                                  _I32, _P, _P, _P]),
    "seer_decode_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(SeerDims), _I32, _I32]),
    "seer_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(SeerDims), _I32, _I32]),
    "seer_decode_num_split": (_I32, [ctypes.POINTER(SeerDims), _I32, _I32, ctypes.POINTER(_I32)]),
    "seer_sparse_decode": (_I32, [ctypes.POINTER(SeerDims), _P, _P, _P, _P, _P, _P, _I32,
                                  ctypes.c_float, _I32, _P, ctypes.c_size_t, _P, _P, _P]),
    "seer_dense_decode": (_I32, [ctypes.POINTER(SeerDims), _P, _P, _P, _P, ctypes.c_float, _I32,
                                 _P, ctypes.c_size_t, _P, _P, _P]),
    "seer_sparse_decode_paged": (_I32, [ctypes.POINTER(SeerDims), _P, _P, _P, ctypes.c_int64,
                                        ctypes.c_int64, _I32, _P, _I32, _P, _P, _P, _I32,
                                        ctypes.c_float, _I32, _P, ctypes.c_size_t, _P, _P, _P]),
    "seer_dense_decode_paged": (_I32, [ctypes.POINTER(SeerDims), _P, _P, _P, ctypes.c_int64,
                                       ctypes.c_int64, _I32, _P, _I32, _P, ctypes.c_float, _I32,
                                       _P, ctypes.c_size_t, _P, _P, _P]),
    "seer_prefill_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(SeerDims)]),
    "seer_prefill_attention": (_I32, [ctypes.POINTER(SeerDims), _P, _P, _P, _P, ctypes.c_float, _P,
                                      ctypes.c_size_t, _P, _P, _P, _P]),
    "seer_decode_step_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(SeerDims), _I32, _I32]),
    "seer_decode_step": (_I32, [ctypes.POINTER(SeerDims), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                _I32, ctypes.c_double, _I32, _I32, ctypes.c_float, _I32, _P, _P,
                                _P, ctypes.c_float, _I32, _P, ctypes.c_size_t, _P, _P, _P]),
    "seer_decode_step_noalloc": (_I32, [ctypes.POINTER(SeerDims), _P, _P, _P, _P, _P, _P, _P,
                                        _P, _P, _P, _I32, ctypes.c_double, _I32, _I32,
                                        ctypes.c_float, _I32, _P, _P, _P, ctypes.c_float, _I32,
                                        _P, _P, _P]),
    "seer_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "seer_last_error_message": (ctypes.c_char_p, []),
    "seer_version": (ctypes.c_char_p, []),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libseer.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -m block_sparse_attention_seer_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def seer_status_string(code: int) -> str:
    return lib().seer_status_string(int(code)).decode()


def seer_last_error_message() -> str:
    return lib().seer_last_error_message().decode()


def seer_version() -> str:
    return lib().seer_version().decode()


def _check(code: int, where: str) -> None:
    if code != SEER_OK:
        raise SeerError(code, where, seer_last_error_message())


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, name: str, dtype, shape=None, device=None, contiguous=True) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def make_dims(batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int, d_gate: int,
              block_size: int, max_seq_len: int, kv_strides=None) -> SeerDims:
    """seer_dims for a [B, H_kv, Lmax, d] KV cache (contiguous unless strides given)."""
    if kv_strides is None:
        kv_strides = (num_kv_heads * max_seq_len * head_dim, max_seq_len * head_dim, head_dim)
    return SeerDims(batch, num_q_heads, num_kv_heads, head_dim, d_gate, block_size, max_seq_len,
                    0, *[int(s) for s in kv_strides])


def _check_kv(dims: SeerDims, t: torch.Tensor, name: str) -> None:
    _need(t, name, torch.bfloat16, contiguous=False)
    if t.dim() != 4 or t.shape[0] != dims.batch or t.shape[1] != dims.num_kv_heads \
            or t.shape[2] < dims.max_seq_len or t.shape[3] != dims.head_dim:
        raise ValueError(f"{name} must be [B, H_kv, >= Lmax, d], got {tuple(t.shape)}")
    if t.stride(3) != 1 or (t.stride(0), t.stride(1), t.stride(2)) != (
            dims.kv_stride_b, dims.kv_stride_h, dims.kv_stride_t):
        raise ValueError(f"{name} strides {t.stride()} do not match dims")


def seer_kcomp_update(dims: SeerDims, k_nope, w_k, seq_lens, kcomp_lens, kcomp,
                      max_new_blocks: int = 1, rope_theta: float = 10000.0) -> None:
    B, Hkv, d, dg = dims.batch, dims.num_kv_heads, dims.head_dim, dims.d_gate
    _check_kv(dims, k_nope, "k_nope")
    dev = k_nope.device
    _need(w_k, "w_k", torch.bfloat16, (Hkv, dg, 3 * d), dev)
    _need(seq_lens, "seq_lens", torch.int32, (B,), dev)
    _need(kcomp_lens, "kcomp_lens", torch.int32, (B,), dev)
    _need(kcomp, "kcomp", torch.bfloat16, (B, Hkv, dims.nb_max, dg), dev)
    _check(lib().seer_kcomp_update(ctypes.byref(dims), _ptr(k_nope), _ptr(w_k), _ptr(seq_lens),
                                   _ptr(kcomp_lens), _ptr(kcomp), int(max_new_blocks),
                                   float(rope_theta), _stream(k_nope)), "seer_kcomp_update")


def seer_gate_workspace_bytes(dims: SeerDims) -> int:
    return int(lib().seer_gate_workspace_bytes(ctypes.byref(dims)))


def seer_gate_scores(dims: SeerDims, q_nope, w_q, kcomp, kcomp_lens, seq_lens, workspace,
                     logits, rope_theta: float = 10000.0) -> None:
    B, Hq, Hkv, d, dg = dims.batch, dims.num_q_heads, dims.num_kv_heads, dims.head_dim, dims.d_gate
    dev = q_nope.device
    _need(q_nope, "q_nope", torch.bfloat16, (B, Hq, d), dev)
    _need(w_q, "w_q", torch.bfloat16, (Hkv, dg, dims.group * d), dev)
    _need(kcomp, "kcomp", torch.bfloat16, (B, Hkv, dims.nb_max, dg), dev)
    _need(kcomp_lens, "kcomp_lens", torch.int32, (B,), dev)
    _need(seq_lens, "seq_lens", torch.int32, (B,), dev)
    _need(logits, "logits", torch.float32, (B, Hkv, dims.nb_max), dev)
    _need(workspace, "workspace", workspace.dtype, None, dev)
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib().seer_gate_scores(ctypes.byref(dims), _ptr(q_nope), _ptr(w_q), _ptr(kcomp),
                                  _ptr(kcomp_lens), _ptr(seq_lens), float(rope_theta),
                                  _ptr(workspace), nbytes, _ptr(logits), _stream(q_nope)),
           "seer_gate_scores")


def seer_select_blocks(dims: SeerDims, logits, kcomp_lens, seq_lens, mode: int, topk_blocks: int,
                       threshold: float, max_selected: int, block_idx, num_selected) -> None:
    B, Hkv = dims.batch, dims.num_kv_heads
    dev = logits.device
    _need(logits, "logits", torch.float32, (B, Hkv, dims.nb_max), dev)
    _need(kcomp_lens, "kcomp_lens", torch.int32, (B,), dev)
    _need(seq_lens, "seq_lens", torch.int32, (B,), dev)
    _need(block_idx, "block_idx", torch.int32, (B, Hkv, max_selected), dev)
    _need(num_selected, "num_selected", torch.int32, (B, Hkv), dev)
    _check(lib().seer_select_blocks(ctypes.byref(dims), _ptr(logits), _ptr(kcomp_lens),
                                    _ptr(seq_lens), int(mode), int(topk_blocks), float(threshold),
                                    int(max_selected), _ptr(block_idx), _ptr(num_selected),
                                    _stream(logits)), "seer_select_blocks")


def seer_workspace_bytes(dims: SeerDims, max_blocks: int, num_split: int = 0) -> int:
    return int(lib().seer_workspace_bytes(ctypes.byref(dims), int(max_blocks), int(num_split)))


def seer_decode_workspace_bytes(dims: SeerDims, max_blocks: int, num_split: int = 0) -> int:
    return int(lib().seer_decode_workspace_bytes(ctypes.byref(dims), int(max_blocks), int(num_split)))


def seer_decode_num_split(dims: SeerDims, max_blocks: int, num_split: int = 0) -> int:
    out = ctypes.c_int32(0)
    _check(lib().seer_decode_num_split(ctypes.byref(dims), int(max_blocks), int(num_split),
                                       ctypes.byref(out)), "seer_decode_num_split")
    return int(out.value)


def _check_decode_io(dims, q, k_cache, v_cache, seq_lens, out, lse):
    B, Hq, d = dims.batch, dims.num_q_heads, dims.head_dim
    dev = q.device
    _need(q, "q", torch.bfloat16, (B, Hq, d), dev)
    _check_kv(dims, k_cache, "k_cache")
    _check_kv(dims, v_cache, "v_cache")
    _need(seq_lens, "seq_lens", torch.int32, (B,), dev)
    _need(out, "out", torch.bfloat16, (B, Hq, d), dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, (B, Hq), dev)


def _ws(workspace, dev):
    if workspace is None:
        return None, 0
    _need(workspace, "workspace", workspace.dtype, None, dev)
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def seer_sparse_decode(dims: SeerDims, q, k_cache, v_cache, seq_lens, block_idx, num_selected,
                       max_selected: int, scale: float, num_split: int, workspace, out,
                       lse=None) -> None:
    _check_decode_io(dims, q, k_cache, v_cache, seq_lens, out, lse)
    dev = q.device
    _need(block_idx, "block_idx", torch.int32, (dims.batch, dims.num_kv_heads, max_selected), dev)
    _need(num_selected, "num_selected", torch.int32, (dims.batch, dims.num_kv_heads), dev)
    wp, wn = _ws(workspace, dev)
    _check(lib().seer_sparse_decode(ctypes.byref(dims), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                    _ptr(seq_lens), _ptr(block_idx), _ptr(num_selected),
                                    int(max_selected), float(scale), int(num_split), wp, wn,
                                    _ptr(out), _ptr(lse), _stream(q)), "seer_sparse_decode")


def seer_dense_decode(dims: SeerDims, q, k_cache, v_cache, seq_lens, scale: float, num_split: int,
                      workspace, out, lse=None) -> None:
    _check_decode_io(dims, q, k_cache, v_cache, seq_lens, out, lse)
    wp, wn = _ws(workspace, q.device)
    _check(lib().seer_dense_decode(ctypes.byref(dims), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                   _ptr(seq_lens), float(scale), int(num_split), wp, wn, _ptr(out),
                                   _ptr(lse), _stream(q)), "seer_dense_decode")


def _check_pages(dims: SeerDims, q, k_pages, v_pages, block_table, seq_lens, out, lse):
    """Page pools [num_pages, H_kv, b, d] bf16 (contiguous) and the block table
    [B, table_stride] int32; returns (num_pages, page_stride, page_head_stride,
    table_stride)."""
    B, Hq, Hkv, d, bs = dims.batch, dims.num_q_heads, dims.num_kv_heads, dims.head_dim, dims.block_size
    dev = q.device
    _need(q, "q", torch.bfloat16, (B, Hq, d), dev)
    if not isinstance(k_pages, torch.Tensor) or k_pages.dim() != 4:
        raise ValueError("k_pages must be a [num_pages, H_kv, block_size, d] tensor")
    num_pages = k_pages.shape[0]
    _need(k_pages, "k_pages", torch.bfloat16, (num_pages, Hkv, bs, d), dev)
    _need(v_pages, "v_pages", torch.bfloat16, (num_pages, Hkv, bs, d), dev)
    if dims.kv_stride_t != d:
        raise ValueError("paged decode: dims.kv_stride_t must be head_dim (rows of a page)")
    if not isinstance(block_table, torch.Tensor) or block_table.dim() != 2:
        raise ValueError("block_table must be a [B, table_stride] int32 tensor")
    _need(block_table, "block_table", torch.int32, (B, block_table.shape[1]), dev)
    _need(seq_lens, "seq_lens", torch.int32, (B,), dev)
    _need(out, "out", torch.bfloat16, (B, Hq, d), dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, (B, Hq), dev)
    return num_pages, Hkv * bs * d, bs * d, block_table.shape[1]


def seer_sparse_decode_paged(dims: SeerDims, q, k_pages, v_pages, block_table, seq_lens,
                             block_idx, num_selected, max_selected: int, scale: float,
                             num_split: int, workspace, out, lse=None) -> None:
    npg, ps, phs, ts = _check_pages(dims, q, k_pages, v_pages, block_table, seq_lens, out, lse)
    dev = q.device
    _need(block_idx, "block_idx", torch.int32, (dims.batch, dims.num_kv_heads, max_selected), dev)
    _need(num_selected, "num_selected", torch.int32, (dims.batch, dims.num_kv_heads), dev)
    wp, wn = _ws(workspace, dev)
    _check(lib().seer_sparse_decode_paged(
        ctypes.byref(dims), _ptr(q), _ptr(k_pages), _ptr(v_pages), ps, phs, npg, _ptr(block_table),
        ts, _ptr(seq_lens), _ptr(block_idx), _ptr(num_selected), int(max_selected), float(scale),
        int(num_split), wp, wn, _ptr(out), _ptr(lse), _stream(q)), "seer_sparse_decode_paged")


def seer_dense_decode_paged(dims: SeerDims, q, k_pages, v_pages, block_table, seq_lens,
                            scale: float, num_split: int, workspace, out, lse=None) -> None:
    npg, ps, phs, ts = _check_pages(dims, q, k_pages, v_pages, block_table, seq_lens, out, lse)
    wp, wn = _ws(workspace, q.device)
    _check(lib().seer_dense_decode_paged(
        ctypes.byref(dims), _ptr(q), _ptr(k_pages), _ptr(v_pages), ps, phs, npg, _ptr(block_table),
        ts, _ptr(seq_lens), float(scale), int(num_split), wp, wn, _ptr(out), _ptr(lse), _stream(q)),
        "seer_dense_decode_paged")


def seer_prefill_workspace_bytes(dims: SeerDims) -> int:
    return int(lib().seer_prefill_workspace_bytes(ctypes.byref(dims)))


def seer_prefill_attention(dims: SeerDims, q, k, v, seq_lens, scale: float, workspace, out, lse,
                           gt=None) -> None:
    """Causal prefill of whole sequences: q, out [B, H_q, Lmax, d] bf16, k, v
    the [B, H_kv, Lmax, d] caches of `dims`, lse [B, H_q, Lmax] float32, gt
    [B, H_kv, Lmax, NBmax] float32 or None."""
    B, Hq, Hkv, d, L = dims.batch, dims.num_q_heads, dims.num_kv_heads, dims.head_dim, dims.max_seq_len
    dev = q.device
    _need(q, "q", torch.bfloat16, (B, Hq, L, d), dev)
    _check_kv(dims, k, "k")
    _check_kv(dims, v, "v")
    _need(seq_lens, "seq_lens", torch.int32, (B,), dev)
    _need(out, "out", torch.bfloat16, (B, Hq, L, d), dev)
    _need(lse, "lse", torch.float32, (B, Hq, L), dev)
    if gt is not None:
        _need(gt, "gt", torch.float32, (B, Hkv, L, dims.nb_max), dev)
    wp, wn = _ws(workspace, dev)
    _check(lib().seer_prefill_attention(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v),
                                        _ptr(seq_lens), float(scale), wp, wn, _ptr(out), _ptr(lse),
                                        _ptr(gt), _stream(q)), "seer_prefill_attention")


def seer_decode_step_workspace_bytes(dims: SeerDims, max_selected: int, num_split: int = 0) -> int:
    return int(lib().seer_decode_step_workspace_bytes(ctypes.byref(dims), int(max_selected),
                                                      int(num_split)))


def seer_decode_step(dims: SeerDims, q_nope, q, k_nope, k_cache, v_cache, w_q, w_k, seq_lens,
                     kcomp_lens, kcomp, max_new_blocks: int, rope_theta: float, mode: int,
                     topk_blocks: int, threshold: float, max_selected: int, block_idx,
                     num_selected, logits, scale: float, num_split: int, workspace, out,
                     lse=None) -> None:
    args = _decode_step_args(dims, q_nope, q, k_nope, k_cache, v_cache, w_q, w_k, seq_lens,
                             kcomp_lens, kcomp, max_new_blocks, rope_theta, mode, topk_blocks,
                             threshold, max_selected, block_idx, num_selected, logits, scale,
                             num_split, workspace, out, lse)
    _check(lib().seer_decode_step(*args, _stream(q)), "seer_decode_step")


def seer_decode_step_noalloc(dims: SeerDims, q_nope, q, k_nope, k_cache, v_cache, w_q, w_k,
                             seq_lens, kcomp_lens, kcomp, max_new_blocks: int, rope_theta: float,
                             mode: int, topk_blocks: int, threshold: float, max_selected: int,
                             block_idx, num_selected, logits, scale: float, num_split: int, out,
                             lse=None) -> None:
    """seer_decode_step with the library's static workspace (no workspace
    argument, nothing allocated by the call)."""
    args = _decode_step_args(dims, q_nope, q, k_nope, k_cache, v_cache, w_q, w_k, seq_lens,
                             kcomp_lens, kcomp, max_new_blocks, rope_theta, mode, topk_blocks,
                             threshold, max_selected, block_idx, num_selected, logits, scale,
                             num_split, None, out, lse)
    args = args[:22] + args[24:]  # without the workspace pointer and size
    _check(lib().seer_decode_step_noalloc(*args, _stream(q)), "seer_decode_step_noalloc")


def _decode_step_args(dims: SeerDims, q_nope, q, k_nope, k_cache, v_cache, w_q, w_k, seq_lens,
                      kcomp_lens, kcomp, max_new_blocks, rope_theta, mode, topk_blocks, threshold,
                      max_selected, block_idx, num_selected, logits, scale, num_split, workspace,
                      out, lse) -> tuple:
    """Checks seer_decode_step's tensors; returns its arguments but the stream."""
    B, Hq, Hkv, d, dg = dims.batch, dims.num_q_heads, dims.num_kv_heads, dims.head_dim, dims.d_gate
    dev = q.device
    _check_decode_io(dims, q, k_cache, v_cache, seq_lens, out, lse)
    _need(q_nope, "q_nope", torch.bfloat16, (B, Hq, d), dev)
    _check_kv(dims, k_nope, "k_nope")
    _need(w_q, "w_q", torch.bfloat16, (Hkv, dg, dims.group * d), dev)
    _need(w_k, "w_k", torch.bfloat16, (Hkv, dg, 3 * d), dev)
    _need(kcomp_lens, "kcomp_lens", torch.int32, (B,), dev)
    _need(kcomp, "kcomp", torch.bfloat16, (B, Hkv, dims.nb_max, dg), dev)
    _need(block_idx, "block_idx", torch.int32, (B, Hkv, max_selected), dev)
    _need(num_selected, "num_selected", torch.int32, (B, Hkv), dev)
    if logits is not None:  # optional: the selection reads the logits from LDS
        _need(logits, "logits", torch.float32, (B, Hkv, dims.nb_max), dev)
    wp, wn = _ws(workspace, dev)
    return (ctypes.byref(dims), _ptr(q_nope), _ptr(q), _ptr(k_nope), _ptr(k_cache), _ptr(v_cache),
            _ptr(w_q), _ptr(w_k), _ptr(seq_lens), _ptr(kcomp_lens), _ptr(kcomp),
            int(max_new_blocks), float(rope_theta), int(mode), int(topk_blocks), float(threshold),
            int(max_selected), _ptr(block_idx), _ptr(num_selected), _ptr(logits), float(scale),
            int(num_split), wp, wn, _ptr(out), _ptr(lse))


class DecodeStep:
    """Buffers and calls of one layer's decode step (allocation via torch).

    Holds the K Compression Cache (kcomp, kcomp_lens), the logits, the index
    tensor, the outputs and three workspaces (gate, decode, fused step).
    ``step`` runs the staged calls (kcomp update, gate, select, sparse
    decode) on the current stream; ``fused_step``, ``bind_step`` and
    ``capture_step`` run the same step through seer_decode_step.  The
    workspaces are zero-filled once here, as the ABI requires of the decode
    counters.
    """

    def __init__(self, dims: SeerDims, *, mode: int, topk_blocks: int = 0, threshold: float = 0.0,
                 max_selected: Optional[int] = None, num_split: int = 0,
                 rope_theta: float = 10000.0, device="cuda"):
        self.dims = dims
        self.mode = int(mode)
        self.topk_blocks = int(topk_blocks)
        self.threshold = float(threshold)
        nbm = dims.nb_max
        if max_selected is None:
            max_selected = (nbm if self.mode in (SELECT_THRESHOLD, SELECT_TOPP)
                            else min(self.topk_blocks + 1, nbm))
        self.max_selected = int(max_selected)
        self.rope_theta = float(rope_theta)
        self.device = torch.device(device)
        B, Hq, Hkv, dg = dims.batch, dims.num_q_heads, dims.num_kv_heads, dims.d_gate
        dev = self.device
        self.kcomp = torch.zeros((B, Hkv, nbm, dg), dtype=torch.bfloat16, device=dev)
        self.kcomp_lens = torch.zeros((B,), dtype=torch.int32, device=dev)
        self.logits = torch.empty((B, Hkv, nbm), dtype=torch.float32, device=dev)
        self.block_idx = torch.empty((B, Hkv, self.max_selected), dtype=torch.int32, device=dev)
        self.num_selected = torch.empty((B, Hkv), dtype=torch.int32, device=dev)
        gws = seer_gate_workspace_bytes(dims)
        self.gate_ws = torch.zeros((max(gws, 16) // 4 + 4,), dtype=torch.float32, device=dev)
        # the caller's request (0 = automatic) goes to the fused step, which
        # may then divide uneven selections evenly over the grid (stream-K);
        # the staged decode calls use the resolved split count
        self.split_request = int(num_split)
        self.num_split = seer_decode_num_split(dims, self.max_selected, num_split)
        # the staged decode's split argument: threshold and top-p with an
        # automatic count take the balanced division, as the fused step does
        # (so both give the same bits); top-k keeps the resolved count
        self.decode_split = (SPLIT_BALANCED if self.mode != SELECT_TOPK
                             and self.split_request in (0, SPLIT_BALANCED) else self.num_split)
        dws = seer_decode_workspace_bytes(dims, self.max_selected, self.decode_split)
        self.decode_ws = torch.zeros((max(dws, 256) // 4 + 64,), dtype=torch.float32, device=dev)
        self.out = torch.empty((B, Hq, dims.head_dim), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
        sws = seer_decode_step_workspace_bytes(dims, self.max_selected, self.split_request)
        self.step_ws = torch.zeros((max(sws, 256) // 4 + 64,), dtype=torch.float32, device=dev)

    @property
    def q_gate(self) -> torch.Tensor:
        d = self.dims
        return self.gate_ws[: d.batch * d.num_kv_heads * d.d_gate].view(d.batch, d.num_kv_heads, d.d_gate)

    def build_cache(self, k_nope, w_k, seq_lens) -> None:
        """Bulk-build every complete block's entry (prompt prefill)."""
        self.kcomp_lens.zero_()
        seer_kcomp_update(self.dims, k_nope, w_k, seq_lens, self.kcomp_lens, self.kcomp,
                          self.dims.nb_max, self.rope_theta)

    def step(self, q_nope, q, k_nope, k_cache, v_cache, w_q, w_k, seq_lens,
             scale: Optional[float] = None, update_cache: bool = True, max_new_blocks: int = 1):
        """The step as four staged calls (cache update of at most
        max_new_blocks entries per pair, gate scores, selection, decode)."""
        d = self.dims
        if scale is None:
            scale = 1.0 / math.sqrt(d.head_dim)
        if update_cache:
            seer_kcomp_update(d, k_nope, w_k, seq_lens, self.kcomp_lens, self.kcomp,
                              int(max_new_blocks), self.rope_theta)
        seer_gate_scores(d, q_nope, w_q, self.kcomp, self.kcomp_lens, seq_lens, self.gate_ws,
                         self.logits, self.rope_theta)
        seer_select_blocks(d, self.logits, self.kcomp_lens, seq_lens, self.mode, self.topk_blocks,
                           self.threshold, self.max_selected, self.block_idx, self.num_selected)
        seer_sparse_decode(d, q, k_cache, v_cache, seq_lens, self.block_idx, self.num_selected,
                           self.max_selected, scale, self.decode_split, self.decode_ws, self.out,
                           self.lse)
        return self.out, self.lse

    def capture_step(self, q_nope, q, k_nope, k_cache, v_cache, w_q, w_k, seq_lens,
                     scale: Optional[float] = None, max_new_blocks: int = 1,
                     keep_logits: bool = False) -> "torch.cuda.CUDAGraph":
        """Records one fused step on these buffers into a HIP graph.

        ``graph.replay()`` then runs the step on the buffers' contents at
        replay time (the caller updates them in place, e.g. appends a token
        and bumps seq_lens), with no host work per step.  The step records
        no memory sets and leaves its split counters at zero, so replays are
        independent.  One eager step runs first (library set-up happens
        outside the capture); it leaves the same state a replay would.
        """
        self.fused_step(q_nope, q, k_nope, k_cache, v_cache, w_q, w_k, seq_lens, scale,
                        max_new_blocks, keep_logits)
        torch.cuda.synchronize(self.device)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            self.fused_step(q_nope, q, k_nope, k_cache, v_cache, w_q, w_k, seq_lens, scale,
                            max_new_blocks, keep_logits)
        return graph

    def bind_step(self, q_nope, q, k_nope, k_cache, v_cache, w_q, w_k, seq_lens,
                  scale: Optional[float] = None, max_new_blocks: int = 1,
                  keep_logits: bool = False):
        """Checks the fused step's tensors once and returns a callable that
        issues the same seer_decode_step with them on the current stream.

        For loops where the per-call checks of this binding would cost more
        host time than the step's GPU work.  The tensors must stay alive and
        in place (the callable holds them); their contents may change between
        calls, as with ``capture_step``.
        """
        d = self.dims
        if scale is None:
            scale = 1.0 / math.sqrt(d.head_dim)
        keep = (q_nope, q, k_nope, k_cache, v_cache, w_q, w_k, seq_lens)
        args = _decode_step_args(d, q_nope, q, k_nope, k_cache, v_cache, w_q, w_k, seq_lens,
                                 self.kcomp_lens, self.kcomp, max_new_blocks, self.rope_theta,
                                 self.mode, self.topk_blocks, self.threshold, self.max_selected,
                                 self.block_idx, self.num_selected,
                                 self.logits if keep_logits else None, scale, self.split_request,
                                 self.step_ws, self.out, self.lse)
        fn = lib().seer_decode_step
        dev = q.device

        def run() -> None:
            _check(fn(*args, torch.cuda.current_stream(dev).cuda_stream), "seer_decode_step")

        run.tensors = keep  # kept alive with the callable
        return run

    def fused_step(self, q_nope, q, k_nope, k_cache, v_cache, w_q, w_k, seq_lens,
                   scale: Optional[float] = None, max_new_blocks: int = 1,
                   keep_logits: bool = True):
        """The same step through seer_decode_step (fewer launches); with
        keep_logits=False the logits are not written out."""
        d = self.dims
        if scale is None:
            scale = 1.0 / math.sqrt(d.head_dim)
        seer_decode_step(d, q_nope, q, k_nope, k_cache, v_cache, w_q, w_k, seq_lens,
                         self.kcomp_lens, self.kcomp, max_new_blocks, self.rope_theta, self.mode,
                         self.topk_blocks, self.threshold, self.max_selected, self.block_idx,
                         self.num_selected, self.logits if keep_logits else None, scale,
                         self.split_request, self.step_ws, self.out, self.lse)
        return self.out, self.lse
