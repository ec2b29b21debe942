"""Python names for the C-ABI calls: argument marshalling only.

Tensors are passed by device pointer and the work is queued on torch's current HIP
stream (or the stream given). Every step of the computation runs in the library's
kernels; a status other than PSD_OK raises PsdError.
"""
from __future__ import annotations

import ctypes

import torch

from . import _native
from ._native import PSD_BF16, PSD_F32, PsdShape

__all__ = ["PsdError", "PsdShape", "make_shape", "page_meta_update", "select_workspace_bytes",
           "select_pages", "decode_workspace_bytes", "sparse_decode", "dense_decode",
           "status_string", "version"]


class PsdError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__(f"{call}: {_native.STATUS.get(status, status)} "
                         f"({status_string(status)})")


def status_string(status: int) -> str:
    return _native.lib().psd_status_string(status).decode()


def version() -> int:
    return _native.lib().psd_version()


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return PSD_BF16
    if t == torch.float32:
        return PSD_F32
    raise TypeError(f"unsupported dtype {t}")


def make_shape(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
               block_table: torch.Tensor, head_dim_v: int | None = None) -> PsdShape:
    """psd_shape for q [B, H_q, D] and caches [num_blocks, 16, H_kv, D(v)] (any strides with
    a contiguous last axis; V may be a leading-dims view of a latent K)."""
    B, Hq, D = q.shape
    NB, page, Hkv, _ = k_cache.shape
    dv = v_cache.shape[-1] if head_dim_v is None else head_dim_v
    ks, vs = k_cache.stride(), v_cache.stride()
    return PsdShape(batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, head_dim_v=dv,
                    page_size=page, num_blocks=NB, max_pages_per_seq=block_table.shape[1],
                    dtype=_dtype_code(q.dtype), reserved=0, k_block_stride=ks[0],
                    k_token_stride=ks[1], k_head_stride=ks[2], v_block_stride=vs[0],
                    v_token_stride=vs[1], v_head_stride=vs[2])


def _ptr(t):
    """Device address of a tensor: device memory as is; pinned host memory (a CPU tensor
    allocated with pin_memory=True) through its device mapping, so that kernels read it
    over the host link. Any other CPU tensor is refused."""
    if t is None:
        return None
    if t.device.type == "cpu":
        if not t.is_pinned():
            raise PsdError(-1, "a host tensor passed to the library must be pinned")
        base = t.untyped_storage().data_ptr()
        return ctypes.c_void_p(_native.host_device_pointer(base) + (t.data_ptr() - base))
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ok(status: int, call: str):
    if status != 0:
        raise PsdError(status, call)


def page_meta_update(shape: PsdShape, k_cache, meta, block_table, seq_lens, first_page=None,
                     stream=None):
    _ok(_native.lib().psd_page_meta_update(ctypes.byref(shape), _ptr(k_cache), _ptr(meta),
                                           _ptr(block_table), _ptr(seq_lens), _ptr(first_page),
                                           _stream(stream)), "psd_page_meta_update")


def select_workspace_bytes(shape: PsdShape, b_max: int) -> int:
    return int(_native.lib().psd_select_workspace_bytes(ctypes.byref(shape), b_max))


def select_pages(shape: PsdShape, q, meta, block_table, seq_lens, budgets, b_max: int, sel_pages,
                 sel_count, workspace, stream=None):
    _ok(_native.lib().psd_select_pages(ctypes.byref(shape), _ptr(q), _ptr(meta),
                                       _ptr(block_table), _ptr(seq_lens), _ptr(budgets), b_max,
                                       _ptr(sel_pages), _ptr(sel_count), _ptr(workspace),
                                       workspace.numel() * workspace.element_size(),
                                       _stream(stream)), "psd_select_pages")


def select_score(shape: PsdShape, q, meta, block_table, seq_lens, budgets, b_max: int, sel_pages,
                 sel_count, workspace, stream=None):
    _ok(_native.lib().psd_select_score(ctypes.byref(shape), _ptr(q), _ptr(meta),
                                       _ptr(block_table), _ptr(seq_lens), _ptr(budgets), b_max,
                                       _ptr(sel_pages), _ptr(sel_count), _ptr(workspace),
                                       workspace.numel() * workspace.element_size(),
                                       _stream(stream)), "psd_select_score")


def select_merge(shape: PsdShape, q, meta, block_table, seq_lens, budgets, b_max: int, sel_pages,
                 workspace, stream=None):
    _ok(_native.lib().psd_select_merge(ctypes.byref(shape), _ptr(q), _ptr(meta),
                                       _ptr(block_table), _ptr(seq_lens), _ptr(budgets), b_max,
                                       _ptr(sel_pages), _ptr(workspace),
                                       workspace.numel() * workspace.element_size(),
                                       _stream(stream)), "psd_select_merge")


def decode_workspace_bytes(shape: PsdShape, max_pages_attended: int) -> int:
    return int(_native.lib().psd_decode_workspace_bytes(ctypes.byref(shape), max_pages_attended))


def sparse_decode(shape: PsdShape, q, k_cache, v_cache, block_table, seq_lens, sel_pages,
                  sel_count, b_max: int, scale: float, out, workspace, stream=None):
    _ok(_native.lib().psd_sparse_decode(ctypes.byref(shape), _ptr(q), _ptr(k_cache),
                                        _ptr(v_cache), _ptr(block_table), _ptr(seq_lens),
                                        _ptr(sel_pages), _ptr(sel_count), b_max, scale,
                                        _ptr(out), _ptr(workspace),
                                        workspace.numel() * workspace.element_size(),
                                        _stream(stream)), "psd_sparse_decode")


def value_tier_state_bytes(shape: PsdShape, slots: int) -> int:
    return int(_native.lib().psd_value_tier_state_bytes(ctypes.byref(shape), slots))


def value_tier_workspace_bytes(shape: PsdShape, b_max: int, slots: int) -> int:
    return int(_native.lib().psd_value_tier_workspace_bytes(ctypes.byref(shape), b_max, slots))


def value_tier_reset(shape: PsdShape, slots: int, state, stream=None):
    _ok(_native.lib().psd_value_tier_reset(ctypes.byref(shape), slots, _ptr(state),
                                           _stream(stream)), "psd_value_tier_reset")


def value_tier_stage(shape: PsdShape, v_host, hot, state, slots: int, step: int, block_table,
                     seq_lens, sel_pages, sel_count, b_max: int, vslot, stats, workspace,
                     stream=None):
    _ok(_native.lib().psd_value_tier_stage(ctypes.byref(shape), _ptr(v_host), _ptr(hot),
                                           _ptr(state), slots, step, _ptr(block_table),
                                           _ptr(seq_lens), _ptr(sel_pages), _ptr(sel_count),
                                           b_max, _ptr(vslot), _ptr(stats), _ptr(workspace),
                                           workspace.numel() * workspace.element_size(),
                                           _stream(stream)), "psd_value_tier_stage")


def sparse_decode_tiered(shape: PsdShape, q, k_cache, v_host, hot, vslot, block_table, seq_lens,
                         sel_pages, sel_count, b_max: int, scale: float, out, workspace,
                         stream=None):
    _ok(_native.lib().psd_sparse_decode_tiered(ctypes.byref(shape), _ptr(q), _ptr(k_cache),
                                               _ptr(v_host), _ptr(hot), _ptr(vslot),
                                               _ptr(block_table), _ptr(seq_lens), _ptr(sel_pages),
                                               _ptr(sel_count), b_max, scale, _ptr(out),
                                               _ptr(workspace),
                                               workspace.numel() * workspace.element_size(),
                                               _stream(stream)), "psd_sparse_decode_tiered")


def kv_tier_stage(shape: PsdShape, k_host, v_host, hot_k, hot_v, state, slots: int, step: int,
                  block_table, seq_lens, sel_pages, sel_count, b_max: int, slot, stats,
                  workspace, stream=None):
    _ok(_native.lib().psd_kv_tier_stage(ctypes.byref(shape), _ptr(k_host), _ptr(v_host),
                                        _ptr(hot_k), _ptr(hot_v), _ptr(state), slots, step,
                                        _ptr(block_table), _ptr(seq_lens), _ptr(sel_pages),
                                        _ptr(sel_count), b_max, _ptr(slot), _ptr(stats),
                                        _ptr(workspace),
                                        workspace.numel() * workspace.element_size(),
                                        _stream(stream)), "psd_kv_tier_stage")


def sparse_decode_kv_tiered(shape: PsdShape, q, k_host, v_host, hot_k, hot_v, slot, block_table,
                            seq_lens, sel_pages, sel_count, b_max: int, scale: float, out,
                            workspace, stream=None):
    _ok(_native.lib().psd_sparse_decode_kv_tiered(
        ctypes.byref(shape), _ptr(q), _ptr(k_host), _ptr(v_host), _ptr(hot_k), _ptr(hot_v),
        _ptr(slot), _ptr(block_table), _ptr(seq_lens), _ptr(sel_pages), _ptr(sel_count), b_max,
        scale, _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)), "psd_sparse_decode_kv_tiered")


def diag_walk(shape: PsdShape, kind: int, k_cache, v_cache, meta, block_table, seq_lens,
              sel_pages, sel_count, b_max: int, checksum, stream=None):
    """Diagnostic: the step's reads with no arithmetic (kind 0: kept K/V rows; kind 1:
    candidate statistics records), XOR-folded per unit into ``checksum`` ([B * H_kv]
    uint32 on the device)."""
    _ok(_native.lib().psd_diag_walk(ctypes.byref(shape), int(kind), _ptr(k_cache), _ptr(v_cache),
                                    _ptr(meta), _ptr(block_table), _ptr(seq_lens),
                                    _ptr(sel_pages), _ptr(sel_count), int(b_max), _ptr(checksum),
                                    _stream(stream)), "psd_diag_walk")


def select_sparse_decode_workspace_bytes(shape: PsdShape, b_max: int) -> int:
    return int(_native.lib().psd_select_sparse_decode_workspace_bytes(ctypes.byref(shape), b_max))


def select_sparse_decode(shape: PsdShape, q, meta, k_cache, v_cache, block_table, seq_lens,
                         budgets, b_max: int, scale: float, sel_pages, sel_count, out, workspace,
                         stream=None):
    _ok(_native.lib().psd_select_sparse_decode(
        ctypes.byref(shape), _ptr(q), _ptr(meta), _ptr(k_cache), _ptr(v_cache),
        _ptr(block_table), _ptr(seq_lens), _ptr(budgets), b_max, scale, _ptr(sel_pages),
        _ptr(sel_count), _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)), "psd_select_sparse_decode")


def decode_step(shape: PsdShape, q, meta, k_cache, v_cache, block_table, seq_lens, budgets,
                b_max: int, scale: float, sel_pages, sel_count, out, workspace, stream=None):
    _ok(_native.lib().psd_decode_step(
        ctypes.byref(shape), _ptr(q), _ptr(meta), _ptr(k_cache), _ptr(v_cache),
        _ptr(block_table), _ptr(seq_lens), _ptr(budgets), b_max, scale, _ptr(sel_pages),
        _ptr(sel_count), _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)), "psd_decode_step")


def decode_step_noalloc(shape: PsdShape, q, meta, k_cache, v_cache, block_table, seq_lens,
                        budgets, b_max: int, scale: float, sel_pages, sel_count, out,
                        stream=None):
    _ok(_native.lib().psd_decode_step_noalloc(
        ctypes.byref(shape), _ptr(q), _ptr(meta), _ptr(k_cache), _ptr(v_cache),
        _ptr(block_table), _ptr(seq_lens), _ptr(budgets), b_max, scale, _ptr(sel_pages),
        _ptr(sel_count), _ptr(out), _stream(stream)), "psd_decode_step_noalloc")


def dense_decode(shape: PsdShape, q, k_cache, v_cache, block_table, seq_lens, scale: float, out,
                 workspace, stream=None):
    _ok(_native.lib().psd_dense_decode(ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                       _ptr(block_table), _ptr(seq_lens), scale, _ptr(out),
                                       _ptr(workspace),
                                       workspace.numel() * workspace.element_size(),
                                       _stream(stream)), "psd_dense_decode")


def select_coverage_workspace_bytes(shape: PsdShape) -> int:
    return int(_native.lib().psd_select_coverage_workspace_bytes(ctypes.byref(shape)))


def select_pages_coverage(shape: PsdShape, q, k_cache, block_table, seq_lens, coverage: float,
                          scale: float, b_max: int, sel_pages, sel_count, workspace, stream=None):
    _ok(_native.lib().psd_select_pages_coverage(
        ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(block_table), _ptr(seq_lens),
        float(coverage), float(scale), int(b_max), _ptr(sel_pages), _ptr(sel_count),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)),
        "psd_select_pages_coverage")

